// C ABI of the retention library: argument validation, per-call planning
// (value tiles, sequence segments, workspace) and kernel dispatch.
// Every check runs on the host before any HIP call, so a rejected call never
// touches the GPU.

#include <math.h>
#include <string.h>

#include "kernels.hpp"

namespace ret {
size_t chunk_f32_lds_bytes(int C, int dk, int dvt);
size_t parallel_f32_lds_bytes(int dk, int dvt);
}  // namespace ret

namespace {

using ret::HeadParams;

constexpr size_t kMaxLdsBytes = 160 * 1024;
constexpr int kTargetBlocks = 256;  // one workgroup per compute unit
constexpr int kMaxSegments = 4096;
constexpr int kMaxAutoSegmentsBf16 = 64;
// The segmented form keeps one ticket counter per (batch, head, value tile)
// chain in a fixed region at the start of the workspace, so counters stay
// counters whatever sizes share the workspace.
constexpr size_t kCtlBytes = 65536;
constexpr long long kMaxSegmentedChains = kCtlBytes / sizeof(unsigned long long);

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ret_status_t fill_head_params(HeadParams& hp, int H, int dk, const float* gamma, const float* theta) {
    memset(&hp, 0, sizeof(hp));
    for (int h = 0; h < H; ++h) {
        if (gamma) {
            const float g = gamma[h];
            if (!(g > 0.0f && g <= 1.0f)) return RET_ERR_GAMMA;  // also rejects NaN
            hp.gamma[h] = g;
        } else {
            hp.gamma[h] = static_cast<float>(1.0 - ldexp(1.0, -5 - h));
        }
    }
    if (theta) {
        for (int j = 0; j < dk / 2; ++j) {
            if (!isfinite(theta[j])) return RET_ERR_GAMMA;
            hp.theta[j] = theta[j];
        }
        hp.has_theta = 1;
    }
    return RET_OK;
}

ret_status_t check_common(int B, int H, int N, int dk, int dv, ret_dtype_t dtype, const float* theta) {
    if (B < 1 || H < 1 || N < 1 || dk < 1 || dv < 1) return RET_ERR_SHAPE;
    if (dtype != RET_F32 && dtype != RET_BF16) return RET_ERR_DTYPE;
    if (theta && (dk % 2) != 0) return RET_ERR_SHAPE;
    if (H > RETENTION_MAX_HEADS) return RET_ERR_UNSUPPORTED;
    if (theta && dk > RETENTION_MAX_DK) return RET_ERR_UNSUPPORTED;
    // element counts must stay well inside size_t / int arithmetic of the kernels
    const double elems = static_cast<double>(B) * H * N * (dk > dv ? dk : dv);
    if (elems > 9.0e15) return RET_ERR_UNSUPPORTED;
    if (static_cast<double>(B) * H * 4096.0 > 2147483647.0) return RET_ERR_UNSUPPORTED;
    return RET_OK;
}

// Value-tile width for the bf16 matrix-core kernels, or 0 if unsupported.
int bf16_dvt(int dk, int dv, int chunk) {
    if (dk != 64 && dk != 128 && dk != 256) return 0;
    if (dv % 64 != 0) return 0;
    if (chunk == 64 && dk == 256) return 64;
    return (dv % 128 == 0) ? 128 : 64;
}

// Value-tile width for the float32 kernels, or 0 if nothing fits in LDS.
int f32_chunk_dvt(int dk, int dv, int chunk) {
    if (dk % 4 != 0 || dv % 16 != 0 || chunk * dk > 8192) return 0;
    for (int w : {64, 32, 16})
        if (dv % w == 0 && ret::chunk_f32_lds_bytes(chunk, dk, w) <= kMaxLdsBytes) return w;
    return 0;
}

int f32_parallel_dvt(int dk, int dv) {
    if (dk % 4 != 0 || dk > 128 || dv % 16 != 0) return 0;
    for (int w : {64, 32, 16})
        if (dv % w == 0 && ret::parallel_f32_lds_bytes(dk, w) <= kMaxLdsBytes) return w;
    return 0;
}

struct ChunkPlan {
    int dvt, nvt, nseg, seg_len, nseg_max;
    size_t ws_bytes;
    int grp;                    // segments per look-back group
    size_t flags_off, gflags_off, agg_off, gagg_off;  // byte offsets of the workspace regions
};

constexpr size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Segment count: enough (batch, head, value tile, segment) workgroups to keep
// every compute unit busy, bounded independently of N so the workspace size
// does not depend on the sequence length.
ret_status_t plan_chunk(int B, int H, int N, int dk, int dv, ret_dtype_t dtype, int chunk, int segments,
                        ChunkPlan& p) {
    if (chunk != 64 && chunk != 128) return RET_ERR_UNSUPPORTED;
    if (segments < 0) return RET_ERR_SHAPE;
    p.dvt = (dtype == RET_BF16) ? bf16_dvt(dk, dv, chunk) : f32_chunk_dvt(dk, dv, chunk);
    if (p.dvt == 0) return RET_ERR_UNSUPPORTED;
    p.nvt = dv / p.dvt;
    const long long base = static_cast<long long>(B) * H * p.nvt;
    if (base > kMaxSegmentedChains)
        p.nseg_max = 1;  // the grid is full without splitting sequences
    else if (segments > 0)
        p.nseg_max = segments;
    else if (base >= 256)
        p.nseg_max = 1;
    else  // each bf16 segment reads every predecessor's state: keep the chains short
        p.nseg_max = static_cast<int>((kTargetBlocks + base - 1) / base);
    if (segments == 0 && dtype == RET_BF16 && p.nseg_max > kMaxAutoSegmentsBf16) p.nseg_max = kMaxAutoSegmentsBf16;
    if (p.nseg_max > kMaxSegments) p.nseg_max = kMaxSegments;
    const int nchunks = (N + chunk - 1) / chunk;
    const int want = p.nseg_max < nchunks ? p.nseg_max : nchunks;
    const int per_seg = (nchunks + want - 1) / want;
    p.seg_len = per_seg * chunk;
    p.nseg = (N + p.seg_len - 1) / p.seg_len;
    // Look-back groups of about sqrt(segments) segments (at least 2): a
    // segment reads its group predecessors' states and one aggregate per
    // earlier group.
    p.grp = 2;
    while ((p.grp + 1) * (p.grp + 1) <= p.nseg) ++p.grp;
    const int ngroups_max = (p.nseg_max + 1) / 2;
    // workspace: [ticket counter per chain | flags per (chain, segment) | flags per (chain, group) |
    //             segment states | group aggregates], chain = (batch, head, value tile)
    const size_t slot = static_cast<size_t>(B) * H * dk * dv * sizeof(float);  // one state per chain
    p.flags_off = kCtlBytes;
    p.gflags_off = p.flags_off + round256(static_cast<size_t>(base) * p.nseg_max * sizeof(unsigned long long));
    p.agg_off = p.gflags_off + round256(static_cast<size_t>(base) * ngroups_max * sizeof(unsigned long long));
    p.gagg_off = p.agg_off + slot * p.nseg_max;
    p.ws_bytes = p.nseg_max > 1 ? p.gagg_off + slot * ngroups_max : 0;
    if (base * p.nseg > 2147483647LL) return RET_ERR_UNSUPPORTED;
    return RET_OK;
}

}  // namespace

extern "C" {

const char* retention_status_string(ret_status_t s) {
    switch (s) {
        case RET_OK: return "ok";
        case RET_ERR_NULL: return "a required pointer is NULL";
        case RET_ERR_SHAPE: return "invalid size (a size < 1, or odd dk with theta)";
        case RET_ERR_DTYPE: return "unknown dtype";
        case RET_ERR_GAMMA: return "gamma outside (0, 1] or non-finite gamma/theta";
        case RET_ERR_UNSUPPORTED: return "valid request outside the implemented set";
        case RET_ERR_WORKSPACE: return "workspace missing or too small";
        case RET_ERR_ALIGN: return "device pointer not 16-byte aligned";
        case RET_ERR_HIP: return "HIP runtime reported a launch error";
    }
    return "unknown status";
}

int retention_abi_version(void) { return RETENTION_ABI_VERSION; }

size_t retention_chunkwise_workspace_size(int B, int H, int N, int dk, int dv, ret_dtype_t dtype, int chunk,
                                          int segments) {
    if (check_common(B, H, N, dk, dv, dtype, nullptr) != RET_OK) return 0;
    ChunkPlan p;
    if (plan_chunk(B, H, N, dk, dv, dtype, chunk, segments, p) != RET_OK) return 0;
    return p.ws_bytes;
}

static ret_status_t chunkwise_impl(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                                   int dk, int dv, ret_dtype_t dtype, int chunk, const float* gamma,
                                   const float* theta, int64_t pos0, const float* state_in, float* state_out,
                                   int segments, void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* events) {
    if (!q || !k || !v || !o) return RET_ERR_NULL;
    ret_status_t s = check_common(B, H, N, dk, dv, dtype, theta);
    if (s != RET_OK) return s;
    if (segments < 0) return RET_ERR_SHAPE;
    HeadParams hp;
    s = fill_head_params(hp, H, dk, gamma, theta);
    if (s != RET_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state_in) ||
        !aligned16(state_out) || !aligned16(workspace))
        return RET_ERR_ALIGN;
    ChunkPlan p;
    s = plan_chunk(B, H, N, dk, dv, dtype, chunk, segments, p);
    if (s != RET_OK) return s;
    if (p.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < p.ws_bytes)) return RET_ERR_WORKSPACE;

    ret::ChunkArgs a;
    a.q = static_cast<const ret::u16*>(q);
    a.k = static_cast<const ret::u16*>(k);
    a.v = static_cast<const ret::u16*>(v);
    a.o = static_cast<ret::u16*>(o);
    a.state_in = state_in;
    a.state_out = state_out;
    char* ws = static_cast<char*>(workspace);
    const bool seg_ws = p.ws_bytes > 0;
    a.ctl = seg_ws ? reinterpret_cast<unsigned long long*>(ws) : nullptr;
    a.flags = seg_ws ? reinterpret_cast<unsigned long long*>(ws + p.flags_off) : nullptr;
    a.agg = seg_ws ? reinterpret_cast<float*>(ws + p.agg_off) : nullptr;
    a.gflags = seg_ws ? reinterpret_cast<unsigned long long*>(ws + p.gflags_off) : nullptr;
    a.gagg = seg_ws ? reinterpret_cast<float*>(ws + p.gagg_off) : nullptr;
    a.B = B;
    a.H = H;
    a.N = N;
    a.dk = dk;
    a.dv = dv;
    a.chunk = chunk;
    a.nvt = p.nvt;
    a.nseg = p.nseg;
    a.seg_len = p.seg_len;
    a.grp = p.grp;
    a.pos0 = pos0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipEvent_t* ev = events ? reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)) : nullptr;
    const hipError_t e = (dtype == RET_BF16) ? ret::launch_chunk_bf16(a, hp, p.dvt, st, ev)
                                             : ret::launch_chunk_f32(a, hp, p.dvt, st, ev);
    return e == hipSuccess ? RET_OK : RET_ERR_HIP;
}

ret_status_t retention_chunkwise_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                                     int dk, int dv, ret_dtype_t dtype, int chunk, const float* gamma,
                                     const float* theta, int64_t pos0, const float* state_in, float* state_out,
                                     int segments, void* workspace, size_t workspace_bytes, void* stream) {
    return chunkwise_impl(q, k, v, o, B, H, N, dk, dv, dtype, chunk, gamma, theta, pos0, state_in, state_out,
                          segments, workspace, workspace_bytes, stream, nullptr);
}

ret_status_t retention_chunkwise_fwd_timed(const void* q, const void* k, const void* v, void* o, int B, int H,
                                           int N, int dk, int dv, ret_dtype_t dtype, int chunk, const float* gamma,
                                           const float* theta, int64_t pos0, const float* state_in,
                                           float* state_out, int segments, void* workspace,
                                           size_t workspace_bytes, void* stream, void* const* events) {
    if (!events) return RET_ERR_NULL;
    for (int i = 0; i < 6; ++i)
        if (!events[i]) return RET_ERR_NULL;
    return chunkwise_impl(q, k, v, o, B, H, N, dk, dv, dtype, chunk, gamma, theta, pos0, state_in, state_out,
                          segments, workspace, workspace_bytes, stream, events);
}

ret_status_t retention_parallel_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                                    int dk, int dv, ret_dtype_t dtype, const float* gamma, const float* theta,
                                    int64_t pos0, void* stream) {
    if (!q || !k || !v || !o) return RET_ERR_NULL;
    ret_status_t s = check_common(B, H, N, dk, dv, dtype, theta);
    if (s != RET_OK) return s;
    HeadParams hp;
    s = fill_head_params(hp, H, dk, gamma, theta);
    if (s != RET_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return RET_ERR_ALIGN;
    const int dvt = (dtype == RET_BF16) ? bf16_dvt(dk, dv, 128) : f32_parallel_dvt(dk, dv);
    if (dvt == 0) return RET_ERR_UNSUPPORTED;
    const long long nqb = (N + 63) / 64;
    if (nqb * B * H * (dv / dvt) > 2147483647LL) return RET_ERR_UNSUPPORTED;

    ret::ParallelArgs a;
    a.q = static_cast<const ret::u16*>(q);
    a.k = static_cast<const ret::u16*>(k);
    a.v = static_cast<const ret::u16*>(v);
    a.o = static_cast<ret::u16*>(o);
    a.B = B;
    a.H = H;
    a.N = N;
    a.dk = dk;
    a.dv = dv;
    a.nvt = dv / dvt;
    a.pos0 = pos0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = (dtype == RET_BF16) ? ret::launch_parallel_bf16(a, hp, dvt, st)
                                             : ret::launch_parallel_f32(a, hp, dvt, st);
    return e == hipSuccess ? RET_OK : RET_ERR_HIP;
}

ret_status_t retention_recurrent_step(const void* q, const void* k, const void* v, void* o, float* state, int B,
                                      int H, int dk, int dv, ret_dtype_t dtype, const float* gamma,
                                      const float* theta, const int64_t* pos, void* stream) {
    if (!q || !k || !v || !o || !state) return RET_ERR_NULL;
    if (theta && !pos) return RET_ERR_NULL;
    ret_status_t s = check_common(B, H, 1, dk, dv, dtype, theta);
    if (s != RET_OK) return s;
    HeadParams hp;
    s = fill_head_params(hp, H, dk, gamma, theta);
    if (s != RET_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state) ||
        !aligned16(pos))
        return RET_ERR_ALIGN;
    if (dv % 4 != 0 || dv > 1024 || dk > 4096) return RET_ERR_UNSUPPORTED;

    ret::StepArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.state = state;
    a.pos = pos;
    a.B = B;
    a.H = H;
    a.dk = dk;
    a.dv = dv;
    a.bf16 = dtype == RET_BF16;
    a.ntile = ret::recurrent_step_tiles(B, H, dv);
    const hipError_t e = ret::launch_recurrent_step(a, hp, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RET_OK : RET_ERR_HIP;
}

}  // extern "C"
