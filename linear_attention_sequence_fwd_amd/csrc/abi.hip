// C ABI of the retention library: argument validation, per-call planning
// (value tiles, sequence segments, workspace) and kernel dispatch.
// Every check runs on the host before any HIP call, so a rejected call never
// touches the GPU.

#include <math.h>
#include <string.h>

#include <mutex>

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
constexpr int kMaxLargeChunk = 1 << 16;
// The segmented form keeps one ticket counter per (batch, head, value tile)
// chain in a fixed region at the start of the workspace, so counters stay
// counters whatever sizes share the workspace; each counter has a 128-byte
// line to itself (the chains' first atomics then do not queue behind each
// other: 16.7 -> 15.9 us on the multi-scale workload), which bounds the
// chains that can be segmented at 512.
constexpr size_t kCtlBytes = 65536;
constexpr long long kMaxSegmentedChains = kCtlBytes / (ret::kCtlStride * sizeof(unsigned long long));

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
    if (chunk == 32 || (chunk == 64 && dk == 256)) return 64;
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
    int tile;  // tokens per kernel chunk (64 or 128): the MFMA tile of the intra-chunk products
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
    // Chunks of 64 or 128 tokens are the kernel's tile. Larger chunks (multiples
    // of 128, bf16) keep the 128-token tile inside the chunk and exchange the
    // state between chunks: one segment per chunk.
    const bool large = chunk > 128;
    if (large ? (dtype != RET_BF16 || chunk % 128 != 0 || chunk > kMaxLargeChunk)
              : (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128))
        return RET_ERR_UNSUPPORTED;
    if (segments < 0) return RET_ERR_SHAPE;
    // bf16 chunks of 16 tokens run as 32-token tiles: the matrix-core contraction
    // over tokens is 32 deep (the chunk length moves only the points where the
    // state is carried, not the result); the float32 kernel takes any chunk
    p.tile = large ? 128 : (chunk == 16 && dtype == RET_BF16 ? 32 : chunk);
    p.dvt = (dtype == RET_BF16) ? bf16_dvt(dk, dv, p.tile) : f32_chunk_dvt(dk, dv, p.tile);
    if (p.dvt == 0) return RET_ERR_UNSUPPORTED;
    p.nvt = dv / p.dvt;
    const long long base = static_cast<long long>(B) * H * p.nvt;
    if (large) {
        const long long nseg = (static_cast<long long>(N) + chunk - 1) / chunk;
        if (nseg > kMaxSegments) return RET_ERR_UNSUPPORTED;
        p.nseg_max = base > kMaxSegmentedChains ? 1 : static_cast<int>(nseg);  // too many chains: one pass
    } else if (base > kMaxSegmentedChains)
        p.nseg_max = 1;  // the grid is full without splitting sequences
    else if (segments > 0)
        p.nseg_max = segments;
    else if (base >= 256)
        p.nseg_max = 1;
    else  // each bf16 segment reads every predecessor's state: keep the chains short
        p.nseg_max = static_cast<int>((kTargetBlocks + base - 1) / base);
    if (!large && segments == 0 && dtype == RET_BF16 && p.nseg_max > kMaxAutoSegmentsBf16)
        p.nseg_max = kMaxAutoSegmentsBf16;
    if (p.nseg_max > kMaxSegments) p.nseg_max = kMaxSegments;
    const int nchunks = (N + p.tile - 1) / p.tile;
    const int want = p.nseg_max < nchunks ? p.nseg_max : nchunks;
    const int per_seg = (nchunks + want - 1) / want;
    p.seg_len = (large && p.nseg_max > 1) ? chunk : per_seg * p.tile;
    p.nseg = (N + p.seg_len - 1) / p.seg_len;
    // the workspace below holds nseg_max segments per chain: the kernels index up to nseg
    if (p.nseg > p.nseg_max) return RET_ERR_UNSUPPORTED;
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
    const size_t flag_bytes = ret::kFlagStride * sizeof(unsigned long long);
    p.gflags_off = p.flags_off + round256(static_cast<size_t>(base) * p.nseg_max * flag_bytes);
    p.agg_off = p.gflags_off + round256(static_cast<size_t>(base) * ngroups_max * flag_bytes);
    p.gagg_off = p.agg_off + slot * p.nseg_max;
    p.ws_bytes = p.nseg_max > 1 ? p.gagg_off + slot * ngroups_max : 0;
    if (base * p.nseg > 2147483647LL) return RET_ERR_UNSUPPORTED;
    return RET_OK;
}

void fill_chunk_args(ret::ChunkArgs& a, const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                     int dk, int dv, int chunk, int64_t pos0, const float* state_in, float* state_out,
                     const ChunkPlan& p, void* workspace) {
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
    a.chunk = p.tile;
    a.nvt = p.nvt;
    a.nseg = p.nseg;
    a.seg_len = p.seg_len;
    a.grp = p.grp;
    a.pos0 = pos0;
    a.rev = 0;
    a.orot = 0;
    a.rescale = 1;
    a.ldqk = 0;
}

// Workspace of the backward: one forward-workspace region per pass first (each
// keeps the zero-filled contract of the forward workspace), then scratch
// tensors. Every pass reads and writes its own buffers, so the passes may run
// concurrently.
struct BwdPlan {
    bool split;                        // bf16 with dv above the key widths: passes 1 and 2 over halves of dv
    int npass;                         // forward passes (3, or 5 when split)
    size_t fwd_bytes;                  // one pass's region; npass of them follow each other from offset 0
    size_t ctl_bytes;                  // leading bytes of each region (counters and flags) cleared per call
    size_t kr, qf, kf, vf, dof;        // [B,H,N,d] rotated / reversed inputs
    size_t dkf, dvf;                   // [B,H,N,d] reversed dK' and dV
    size_t doh, vh;                    // split: halves of dO and V, [B,H,N,dv/2] twice each
    size_t t1, t2;                     // split: second halves' dQ' and dK', [B,H,N,dk]
    size_t x1, x2, x3;                 // float32 [B,H,dk,dv] states
    size_t total;
};

constexpr float kMinBwdGamma = 9.5367431640625e-07f;  // 2^-20: dS / gamma stays far from float32 overflow

ret_status_t plan_bwd(int B, int H, int N, int dk, int dv, ret_dtype_t dtype, int chunk, BwdPlan& b) {
    if (dk % 8 != 0 || dv % 8 != 0) return RET_ERR_UNSUPPORTED;
    ChunkPlan p1, p3;  // passes 1 and 2 have key width dv and value width dk; pass 3 the reverse
    b.split = false;
    ret_status_t s = plan_chunk(B, H, N, dv, dk, dtype, chunk, 0, p1);
    if (s == RET_ERR_UNSUPPORTED && dtype == RET_BF16 && dv % 16 == 0) {
        // dv wider than the matrix-core kernel's keys: run passes 1 and 2 over the halves of dv
        s = plan_chunk(B, H, N, dv / 2, dk, dtype, chunk, 0, p1);
        b.split = s == RET_OK;
    }
    if (s != RET_OK) return s;
    b.npass = b.split ? 5 : 3;
    s = plan_chunk(B, H, N, dk, dv, dtype, chunk, 0, p3);
    if (s != RET_OK) return s;
    const size_t es = dtype == RET_BF16 ? 2 : 4;
    const size_t rows = static_cast<size_t>(B) * H * N;
    const size_t nk = round256(rows * dk * es), nv = round256(rows * dv * es);
    const size_t ns = round256(static_cast<size_t>(B) * H * dk * dv * sizeof(float));
    b.fwd_bytes = round256(p1.ws_bytes > p3.ws_bytes ? p1.ws_bytes : p3.ws_bytes);
    // counters and flags precede the published states in a forward workspace
    const size_t c1 = p1.ws_bytes > 0 ? p1.agg_off : 0, c3 = p3.ws_bytes > 0 ? p3.agg_off : 0;
    b.ctl_bytes = c1 > c3 ? c1 : c3;
    b.kr = static_cast<size_t>(b.npass) * b.fwd_bytes;
    b.qf = b.kr + nk;
    b.kf = b.qf + nk;
    b.vf = b.kf + nk;
    b.dof = b.vf + nv;
    b.dkf = b.dof + nv;
    b.dvf = b.dkf + nk;
    b.doh = b.dvf + nv;
    b.vh = b.doh + (b.split ? nv : 0);
    b.t1 = b.vh + (b.split ? nv : 0);
    b.t2 = b.t1 + (b.split ? nk : 0);
    b.x1 = b.t2 + (b.split ? nk : 0);
    b.x2 = b.x1 + ns;
    b.x3 = b.x2 + ns;
    b.total = b.x3 + ns;
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

ret_status_t retention_chunkwise_plan(int B, int H, int N, int dk, int dv, ret_dtype_t dtype, int chunk,
                                      int segments, ret_chunk_plan_t* out) {
    if (!out) return RET_ERR_NULL;
    ret_status_t s = check_common(B, H, N, dk, dv, dtype, nullptr);
    if (s != RET_OK) return s;
    ChunkPlan p;
    s = plan_chunk(B, H, N, dk, dv, dtype, chunk, segments, p);
    if (s != RET_OK) return s;
    out->tile = p.tile;
    out->dv_tile = p.dvt;
    out->value_tiles = p.nvt;
    out->segments = p.nseg;
    out->segment_len = p.seg_len;
    out->group_len = p.grp;
    out->segments_max = p.nseg_max;
    out->reserved = 0;
    out->flags_off = p.flags_off;
    out->gflags_off = p.gflags_off;
    out->agg_off = p.agg_off;
    out->gagg_off = p.gagg_off;
    out->workspace_bytes = p.ws_bytes;
    return RET_OK;
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
    fill_chunk_args(a, q, k, v, o, B, H, N, dk, dv, chunk, pos0, state_in, state_out, p, workspace);
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

// ---- allocation-free variant: the workspace is a device array of the library
//
// `scratch` holds the segmented form's workspace for retention_chunkwise_fwd_noalloc.
// Static device storage starts zero-filled when the library's code object is
// loaded, which is the state the workspace needs before its first use; every
// call leaves it ready for the next one (counters carry a launch generation),
// so nothing is cleared per call. In host code `scratch` names a host-side
// stand-in: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[RETENTION_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null until looked up)

// The calling thread's current device's copy of `scratch`, or null.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        scratch_ptr[dev] = p;
    }
    return scratch_ptr[dev];
}
}  // namespace

ret_status_t retention_chunkwise_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H,
                                             int N, int dk, int dv, ret_dtype_t dtype, int chunk, const float* gamma,
                                             const float* theta, int64_t pos0, const float* state_in,
                                             float* state_out, int segments, void* stream) {
    if (!q || !k || !v || !o) return RET_ERR_NULL;
    ret_status_t s = check_common(B, H, N, dk, dv, dtype, theta);
    if (s != RET_OK) return s;
    if (segments < 0) return RET_ERR_SHAPE;
    ChunkPlan p;
    s = plan_chunk(B, H, N, dk, dv, dtype, chunk, segments, p);
    if (s != RET_OK) return s;
    if (p.ws_bytes > RETENTION_NOALLOC_SCRATCH_BYTES) return RET_ERR_WORKSPACE;
    void* ws = nullptr;
    if (p.ws_bytes > 0) {
        ws = device_scratch();
        if (!ws) return RET_ERR_HIP;
    }
    return chunkwise_impl(q, k, v, o, B, H, N, dk, dv, dtype, chunk, gamma, theta, pos0, state_in, state_out,
                          segments, ws, p.ws_bytes, stream, nullptr);
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

size_t retention_chunkwise_bwd_workspace_size(int B, int H, int N, int dk, int dv, ret_dtype_t dtype,
                                              int chunk) {
    if (check_common(B, H, N, dk, dv, dtype, nullptr) != RET_OK) return 0;
    if (check_common(B, H, N, dv, dk, dtype, nullptr) != RET_OK) return 0;
    BwdPlan b;
    if (plan_bwd(B, H, N, dk, dv, dtype, chunk, b) != RET_OK) return 0;
    return b.total;
}

ret_status_t retention_chunkwise_bwd(const void* q, const void* k, const void* v, const void* d_o, void* d_q,
                                     void* d_k, void* d_v, int B, int H, int N, int dk, int dv,
                                     ret_dtype_t dtype, int chunk, const float* gamma, const float* theta,
                                     int64_t pos0, const float* state_in, const float* d_state_out,
                                     float* d_state_in, void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !d_o || !d_q || !d_k || !d_v) return RET_ERR_NULL;
    ret_status_t s = check_common(B, H, N, dk, dv, dtype, theta);
    if (s != RET_OK) return s;
    s = check_common(B, H, N, dv, dk, dtype, nullptr);  // dv serves as a key width
    if (s != RET_OK) return s;
    HeadParams hp;
    s = fill_head_params(hp, H, dk, gamma, theta);
    if (s != RET_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(d_q) ||
        !aligned16(d_k) || !aligned16(d_v) || !aligned16(state_in) || !aligned16(d_state_out) ||
        !aligned16(d_state_in) || !aligned16(workspace))
        return RET_ERR_ALIGN;
    BwdPlan b;
    s = plan_bwd(B, H, N, dk, dv, dtype, chunk, b);
    if (s != RET_OK) return s;
    if (d_state_out)
        for (int h = 0; h < H; ++h)
            if (hp.gamma[h] < kMinBwdGamma) return RET_ERR_UNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < b.total) return RET_ERR_WORKSPACE;

    char* ws = static_cast<char*>(workspace);
    void* kr = ws + b.kr;
    void* qf = ws + b.qf;
    void* kf = ws + b.kf;
    void* vf = ws + b.vf;
    void* dof = ws + b.dof;
    void* dkf = ws + b.dkf;
    void* dvf = ws + b.dvf;
    float* x1 = reinterpret_cast<float*>(ws + b.x1);
    float* x2 = reinterpret_cast<float*>(ws + b.x2);
    float* x3 = reinterpret_cast<float*>(ws + b.x3);
    const bool rot = theta != nullptr;
    const bool bf16 = dtype == RET_BF16;
    hipStream_t st = static_cast<hipStream_t>(stream);

    ret::RowJobs rj;
    memset(&rj, 0, sizeof(rj));
    rj.B = B;
    rj.H = H;
    rj.N = N;
    rj.pos0 = pos0;
    // the passes' counters and flags start from zero on every call (the
    // scratch tensors of earlier calls of other sizes may have covered them)
    if (b.ctl_bytes > 0) {
        for (int r = 0; r < b.npass; ++r) rj.zero[r] = reinterpret_cast<uint4*>(ws + r * b.fwd_bytes);
        rj.nzero = static_cast<long long>(b.ctl_bytes / 16);
    }
    const float* sx1 = state_in ? x1 : nullptr;
    const float* sx2 = d_state_out ? x2 : nullptr;
    const float* sx3 = d_state_out ? x3 : nullptr;
    auto prep_states = [&]() -> ret_status_t {
        if (state_in || d_state_out) {
            ret::StateJobs sj = {state_in, d_state_out, x1, x2, x3, nullptr, B, H, dk, dv, 0, b.split ? 1 : 0};
            if (ret::launch_states(sj, hp, st) != hipSuccess) return RET_ERR_HIP;
        }
        return RET_OK;
    };
    auto finish_states = [&]() -> ret_status_t {
        if (d_state_in) {
            ret::StateJobs sj = {nullptr, nullptr, nullptr, nullptr, nullptr, d_state_in, B, H, dk, dv, 1, 0};
            if (ret::launch_states(sj, hp, st) != hipSuccess) return RET_ERR_HIP;
        }
        return RET_OK;
    };

    // The three passes:
    //   dQ' = F(dO, V, K'; S0^T)
    //   dK' = rev F(rev V, rev dO, rev Q'; dS^T / gamma)
    //   dV  = rev F(rev K', rev Q', rev dO; dS / gamma), whose final state is dS0 / gamma
    if (bf16) {
        // The matrix-core kernel reads and writes the reversed passes in
        // reverse token order itself: only the rotation needs copies (K' and
        // Q' in token order) and, at the end, the rotation of dQ', dK' back.
        // With split, the halves of dO and V are copied out as well.
        const int hv = b.split ? dv / 2 : dv;  // key width of passes 1 and 2
        char* doa = ws + b.doh;
        char* dob = doa + static_cast<size_t>(B) * H * N * hv * 2;
        char* va = ws + b.vh;
        char* vb = va + static_cast<size_t>(B) * H * N * hv * 2;
        // 128-token chunks with key widths of 128 or 256 (passes 1 and 2 keyed by hv, pass 3 by
        // dk, equal) and value widths that are multiples of 128: every pass runs on the wide
        // chunkwise kernel, all in one launch, when together they fill the chip; the split
        // passes then read their halves of dO and V in place
        const long long wide_chains = (b.split ? 4LL : 2LL) * B * H * (dk / 128) + 1LL * B * H * (dv / 128);
        const bool wide = chunk == 128 && hv == dk && (dk == 128 || dk == 256) && dv % 128 == 0 &&
                          ret::chunk_wide_rescale(hp, H) > 0 && wide_chains >= kTargetBlocks;
        if (rot) {
            rj.j[rj.n++] = {q, qf, nullptr, dk, 0, 1, 0, 0, 0, nullptr};
            rj.j[rj.n++] = {k, kr, nullptr, dk, 0, 1, 0, 0, 0, nullptr};
        }
        if (b.split && !wide) {
            rj.j[rj.n++] = {d_o, doa, nullptr, hv, 0, 0, 0, dv, 0, nullptr};
            rj.j[rj.n++] = {d_o, dob, nullptr, hv, 0, 0, 0, dv, hv, nullptr};
            rj.j[rj.n++] = {v, va, nullptr, hv, 0, 0, 0, dv, 0, nullptr};
            rj.j[rj.n++] = {v, vb, nullptr, hv, 0, 0, 0, dv, hv, nullptr};
        }
        if (rj.n > 0 || rj.nzero > 0)
            if (ret::launch_rows(rj, hp, bf16, st) != hipSuccess) return RET_ERR_HIP;
        s = prep_states();
        if (s != RET_OK) return s;
        const void* kp = rot ? kr : k;  // K'
        const void* qp = rot ? qf : q;  // Q'
        HeadParams hp_passes = hp;
        hp_passes.has_theta = 0;
        if (wide) {
            ChunkPlan pw;
            memset(&pw, 0, sizeof(pw));
            pw.tile = 128;
            pw.dvt = 128;
            pw.nseg = 1;
            pw.seg_len = N;
            pw.grp = 1;
            auto call = [&](ret::ChunkArgs& a, const void* aq, const void* ak, const void* av, void* ao, int vw,
                            const float* sin, float* sout, int rev, int ldqk) {
                pw.nvt = vw / 128;
                fill_chunk_args(a, aq, ak, av, ao, B, H, N, dk, vw, chunk, 0, sin, sout, pw, nullptr);
                a.rev = rev;
                a.ldqk = ldqk;
            };
            // column block `half` of a [B,H,N,dv] bf16 tensor, read with row stride dv
            auto half_of = [&](const void* t, int half) {
                return static_cast<const void*>(static_cast<const char*>(t) + static_cast<size_t>(half) * hv * 2);
            };
            ret::ChunkCalls cw;
            memset(&cw, 0, sizeof(cw));
            const size_t xh = static_cast<size_t>(B) * H * hv * dk;  // floats in one half of a split state
            if (b.split) {
                call(cw.a[0], half_of(d_o, 0), half_of(v, 0), kp, d_q, dk, sx1, nullptr, 0, dv);
                call(cw.a[1], half_of(d_o, 1), half_of(v, 1), kp, ws + b.t1, dk, sx1 ? sx1 + xh : nullptr, nullptr, 0,
                     dv);
                call(cw.a[2], half_of(v, 0), half_of(d_o, 0), qp, d_k, dk, sx2, nullptr, 1, dv);
                call(cw.a[3], half_of(v, 1), half_of(d_o, 1), qp, ws + b.t2, dk, sx2 ? sx2 + xh : nullptr, nullptr, 1,
                     dv);
                cw.n = 4;
            } else {
                call(cw.a[0], d_o, v, kp, d_q, dk, sx1, nullptr, 0, 0);
                call(cw.a[1], v, d_o, qp, d_k, dk, sx2, nullptr, 1, 0);
                cw.n = 2;
            }
            call(cw.a[cw.n++], kp, qp, d_o, d_v, dv, sx3, d_state_in, 1, 0);
            if (ret::launch_chunk_wide_multi(cw, hp_passes, st) != hipSuccess) return RET_ERR_HIP;
            if (b.split || rot) {  // dQ = R^-1 (dQ'_a + dQ'_b), dK likewise (in place)
                memset(&rj.j, 0, sizeof(rj.j));
                rj.nzero = 0;
                rj.n = 2;
                rj.j[0] = {d_q, d_q, nullptr, dk, 0, rot ? -1 : 0, 0, 0, 0, b.split ? ws + b.t1 : nullptr};
                rj.j[1] = {d_k, d_k, nullptr, dk, 0, rot ? -1 : 0, 0, 0, 0, b.split ? ws + b.t2 : nullptr};
                if (ret::launch_rows(rj, hp, bf16, st) != hipSuccess) return RET_ERR_HIP;
            }
            return finish_states();
        }
        ChunkPlan p1, p3;  // key width hv (passes 1, 2) and dk (pass 3)
        s = plan_chunk(B, H, N, hv, dk, dtype, chunk, 0, p1);
        if (s != RET_OK) return s;
        s = plan_chunk(B, H, N, dk, dv, dtype, chunk, 0, p3);
        if (s != RET_OK) return s;
        // Keys and values of one width (128 or 256) in 128-token chunks whose plan cuts the
        // sequence (few heads): the three passes run on the wide kernel's segmented form
        // (their state passes, scans and segment passes, one launch each for all three),
        // each pass with its own workspace region
        if (!b.split && dk == dv && (dk == 128 || dk == 256) && chunk == 128 && p1.nseg > 1 && p1.tile == 128 &&
            p1.dvt == 128 && ret::chunk_wide_rescale(hp, H) > 0) {
            ret::ChunkCalls cw;
            memset(&cw, 0, sizeof(cw));
            fill_chunk_args(cw.a[0], d_o, v, kp, d_q, B, H, N, dv, dk, chunk, 0, sx1, nullptr, p1, ws);
            fill_chunk_args(cw.a[1], v, d_o, qp, d_k, B, H, N, dv, dk, chunk, 0, sx2, nullptr, p1, ws + b.fwd_bytes);
            fill_chunk_args(cw.a[2], kp, qp, d_o, d_v, B, H, N, dk, dv, chunk, 0, sx3, d_state_in, p3,
                            ws + 2 * b.fwd_bytes);
            cw.a[1].rev = 1;
            cw.a[2].rev = 1;
            cw.n = 3;
            if (ret::launch_chunk_wide_multi(cw, hp_passes, st) != hipSuccess) return RET_ERR_HIP;
            if (rot) {  // dQ = R^-1 dQ', dK likewise (in place)
                memset(&rj.j, 0, sizeof(rj.j));
                rj.nzero = 0;
                rj.n = 2;
                rj.j[0] = {d_q, d_q, nullptr, dk, 0, -1, 0, 0, 0, nullptr};
                rj.j[1] = {d_k, d_k, nullptr, dk, 0, -1, 0, 0, 0, nullptr};
                if (ret::launch_rows(rj, hp, bf16, st) != hipSuccess) return RET_ERR_HIP;
            }
            return finish_states();
        }
        // Split passes whose tile matches pass 3's (hv == dk) share its launch
        // when the five passes together fill the chip without sequence
        // segments (one kernel form for all of them).
        bool together = false;
        if (b.split && hv == dk) {
            ChunkPlan q1, q3;
            if (plan_chunk(B, H, N, hv, dk, dtype, chunk, 1, q1) == RET_OK &&
                plan_chunk(B, H, N, dk, dv, dtype, chunk, 1, q3) == RET_OK && q1.dvt == q3.dvt &&
                4LL * B * H * q1.nvt + static_cast<long long>(B) * H * q3.nvt >= kTargetBlocks) {
                p1 = q1;
                p3 = q3;
                together = true;
            }
        }
        // with rotation and no dv split the first two passes rotate their outputs back when the
        // frequencies fit in LDS beside their tiles; otherwise a row kernel does it afterwards
        const bool orot = rot && !b.split && ret::chunk_orot_fits(dv, p1.dvt, p1.tile);
        ret::ChunkCalls cs;
        ret::ChunkArgs a3;
        const size_t xh = static_cast<size_t>(B) * H * hv * dk;  // floats in one half of a split state
        if (b.split) {
            char* t1 = ws + b.t1;
            char* t2 = ws + b.t2;
            fill_chunk_args(cs.a[0], doa, va, kp, d_q, B, H, N, hv, dk, chunk, 0, sx1, nullptr, p1, ws);
            fill_chunk_args(cs.a[1], dob, vb, kp, t1, B, H, N, hv, dk, chunk, 0, sx1 ? sx1 + xh : nullptr, nullptr,
                            p1, ws + b.fwd_bytes);
            fill_chunk_args(cs.a[2], va, doa, qp, d_k, B, H, N, hv, dk, chunk, 0, sx2, nullptr, p1,
                            ws + 2 * b.fwd_bytes);
            fill_chunk_args(cs.a[3], vb, dob, qp, t2, B, H, N, hv, dk, chunk, 0, sx2 ? sx2 + xh : nullptr, nullptr,
                            p1, ws + 3 * b.fwd_bytes);
            cs.a[2].rev = 1;
            cs.a[3].rev = 1;
            cs.n = 4;
            fill_chunk_args(a3, kp, qp, d_o, d_v, B, H, N, dk, dv, chunk, 0, sx3, d_state_in, p3,
                            ws + 4 * b.fwd_bytes);
        } else {
            fill_chunk_args(cs.a[0], d_o, v, kp, d_q, B, H, N, dv, dk, chunk, 0, sx1, nullptr, p1, ws);
            fill_chunk_args(cs.a[1], v, d_o, qp, d_k, B, H, N, dv, dk, chunk, 0, sx2, nullptr, p1, ws + b.fwd_bytes);
            cs.a[1].rev = 1;
            if (orot) {  // the passes store dQ = R^-1 dQ' and dK = R^-1 dK' themselves
                cs.a[0].orot = cs.a[1].orot = 1;
                cs.a[0].pos0 = cs.a[1].pos0 = pos0;  // positions of the output rotation (has_theta is off)
            }
            cs.n = 2;
            fill_chunk_args(a3, kp, qp, d_o, d_v, B, H, N, dk, dv, chunk, 0, sx3, d_state_in, p3,
                            ws + 2 * b.fwd_bytes);
        }
        a3.rev = 1;
        if ((!b.split && dk == dv) || together) {  // a single launch runs them all side by side
            cs.a[cs.n++] = a3;
            if (ret::launch_chunk_bf16_multi(cs, hp_passes, p1.dvt, st) != hipSuccess) return RET_ERR_HIP;
        } else {
            if (ret::launch_chunk_bf16_multi(cs, hp_passes, p1.dvt, st) != hipSuccess) return RET_ERR_HIP;
            ret::ChunkCalls c3;
            c3.a[0] = a3;
            c3.n = 1;
            if (ret::launch_chunk_bf16_multi(c3, hp_passes, p3.dvt, st) != hipSuccess) return RET_ERR_HIP;
        }
        if (b.split || (rot && !orot)) {  // dQ = R^-1 (dQ'_a + dQ'_b), dK likewise (in place)
            memset(&rj.j, 0, sizeof(rj.j));
            rj.nzero = 0;
            rj.n = 2;
            rj.j[0] = {d_q, d_q, nullptr, dk, 0, rot ? -1 : 0, 0, 0, 0, b.split ? ws + b.t1 : nullptr};
            rj.j[1] = {d_k, d_k, nullptr, dk, 0, rot ? -1 : 0, 0, 0, 0, b.split ? ws + b.t2 : nullptr};
            if (ret::launch_rows(rj, hp, bf16, st) != hipSuccess) return RET_ERR_HIP;
        }
        return finish_states();
    }

    // float32: the passes run on reversed and rotated copies
    rj.n = 4;
    rj.j[0] = {q, qf, nullptr, dk, 1, rot ? 1 : 0, 0, 0, 0, nullptr};
    rj.j[1] = {k, kf, rot ? kr : nullptr, dk, 1, rot ? 1 : 0, 0, 0, 0, nullptr};
    rj.j[2] = {v, vf, nullptr, dv, 1, 0, 0, 0, 0, nullptr};
    rj.j[3] = {d_o, dof, nullptr, dv, 1, 0, 0, 0, 0, nullptr};
    if (ret::launch_rows(rj, hp, bf16, st) != hipSuccess) return RET_ERR_HIP;
    s = prep_states();
    if (s != RET_OK) return s;
    const void* pk = rot ? kr : k;
    s = chunkwise_impl(d_o, v, pk, d_q, B, H, N, dv, dk, dtype, chunk, gamma, nullptr, 0, sx1, nullptr, 0, ws,
                       b.fwd_bytes, stream, nullptr);
    if (s != RET_OK) return s;
    s = chunkwise_impl(vf, dof, qf, dkf, B, H, N, dv, dk, dtype, chunk, gamma, nullptr, 0, sx2, nullptr, 0,
                       ws + b.fwd_bytes, b.fwd_bytes, stream, nullptr);
    if (s != RET_OK) return s;
    s = chunkwise_impl(kf, qf, dof, dvf, B, H, N, dk, dv, dtype, chunk, gamma, nullptr, 0, sx3, d_state_in, 0,
                       ws + 2 * b.fwd_bytes, b.fwd_bytes, stream, nullptr);
    if (s != RET_OK) return s;

    // back to token order and unrotated coordinates
    memset(&rj.j, 0, sizeof(rj.j));
    rj.nzero = 0;
    int n = 0;
    if (rot) rj.j[n++] = {d_q, d_q, nullptr, dk, 0, -1, 0, 0, 0, nullptr};
    rj.j[n++] = {dkf, d_k, nullptr, dk, 1, rot ? -1 : 0, 1, 0, 0, nullptr};
    rj.j[n++] = {dvf, d_v, nullptr, dv, 1, 0, 1, 0, 0, nullptr};
    rj.n = n;
    if (ret::launch_rows(rj, hp, bf16, st) != hipSuccess) return RET_ERR_HIP;
    return finish_states();
}

namespace {

// y = z W_O^T for the output stage, z being the bf16 [B*N, H*dv] block at the start
// of the workspace and the split-K partial sums (when any) after it.
ret_status_t msr_projection(const void* w_o, void* y, int B, int H, int N, int dv, int d_out, void* workspace,
                            hipStream_t st) {
    ret::GemmArgs g;
    g.a = static_cast<const ret::u16*>(workspace);
    g.b = static_cast<const ret::u16*>(w_o);
    g.c = static_cast<ret::u16*>(y);
    g.M = B * N;
    g.N = d_out;
    g.K = H * dv;
    g.splits = ret::gemm_splits(g.M, g.N, g.K);
    g.part = g.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                     round256(static_cast<size_t>(B) * N * H * dv * sizeof(uint16_t)))
                          : nullptr;
    return ret::launch_gemm_bt(g, st) == hipSuccess ? RET_OK : RET_ERR_HIP;
}

ret::StepArgs step_args(const void* q, const void* k, const void* v, void* o, float* state, const int64_t* pos, int B,
                        int H, int dk, int dv, ret_dtype_t dtype) {
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
    a.gate = nullptr;
    a.gn_w = nullptr;
    a.gn_b = nullptr;
    a.z = nullptr;
    a.eps = 0.f;
    return a;
}

}  // namespace

size_t retention_msr_epilogue_workspace_size(int B, int H, int N, int dv, int d_out, ret_dtype_t dtype) {
    if (B < 1 || H < 1 || N < 1 || dv < 1 || d_out < 1 || dtype != RET_BF16) return 0;
    if (dv != 64 && dv != 128 && dv != 256 && dv != 512) return 0;
    if (d_out % 128 != 0 || (static_cast<long long>(H) * dv) % 64 != 0) return 0;
    const double rows = static_cast<double>(B) * N;
    if (rows > 2147483647.0 || rows * H * dv > 9.0e15) return 0;
    const int splits = ret::gemm_splits(B * N, d_out, H * dv);
    const size_t part = splits > 1 ? static_cast<size_t>(splits) * B * N * d_out * sizeof(float) : 0;
    return round256(static_cast<size_t>(B) * N * H * dv * sizeof(uint16_t)) + part;
}

ret_status_t retention_msr_epilogue(const void* o, const void* gate, const float* gn_weight, const float* gn_bias,
                                    float eps, const void* w_o, void* y, int B, int H, int N, int dv, int d_out,
                                    ret_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (!o || !w_o || !y) return RET_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || dv < 1 || d_out < 1) return RET_ERR_SHAPE;
    if (dtype != RET_F32 && dtype != RET_BF16) return RET_ERR_DTYPE;
    if (!(eps >= 0.0f) || !isfinite(eps)) return RET_ERR_GAMMA;
    if (!aligned16(o) || !aligned16(gate) || !aligned16(gn_weight) || !aligned16(gn_bias) || !aligned16(w_o) ||
        !aligned16(y) || !aligned16(workspace))
        return RET_ERR_ALIGN;
    const size_t need = retention_msr_epilogue_workspace_size(B, H, N, dv, d_out, dtype);
    if (need == 0) return RET_ERR_UNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < need) return RET_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    ret::EpilogueArgs a;
    a.o = static_cast<const ret::u16*>(o);
    a.gate = static_cast<const ret::u16*>(gate);
    a.gn_weight = gn_weight;
    a.gn_bias = gn_bias;
    a.z = static_cast<ret::u16*>(workspace);
    a.B = B;
    a.H = H;
    a.N = N;
    a.dv = dv;
    a.eps = eps;
    if (ret::launch_groupnorm_gate(a, st) != hipSuccess) return RET_ERR_HIP;
    return msr_projection(w_o, y, B, H, N, dv, d_out, workspace, st);
}

ret_status_t retention_recurrent_step_msr(const void* q, const void* k, const void* v, float* state, int B, int H,
                                          int dk, int dv, ret_dtype_t dtype, const float* gamma, const float* theta,
                                          const int64_t* pos, const void* gate, const float* gn_weight,
                                          const float* gn_bias, float eps, const void* w_o, int d_out, void* o,
                                          void* y, void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !o || !state || !w_o || !y) return RET_ERR_NULL;
    if (theta && !pos) return RET_ERR_NULL;
    ret_status_t s = check_common(B, H, 1, dk, dv, dtype, theta);
    if (s != RET_OK) return s;
    if (d_out < 1) return RET_ERR_SHAPE;
    HeadParams hp;
    s = fill_head_params(hp, H, dk, gamma, theta);
    if (s != RET_OK) return s;
    if (!(eps >= 0.0f) || !isfinite(eps)) return RET_ERR_GAMMA;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state) || !aligned16(pos) ||
        !aligned16(gate) || !aligned16(gn_weight) || !aligned16(gn_bias) || !aligned16(w_o) || !aligned16(y) ||
        !aligned16(workspace))
        return RET_ERR_ALIGN;
    if (dtype != RET_BF16 || dv % 4 != 0 || dv > 1024 || dk > 4096) return RET_ERR_UNSUPPORTED;
    const size_t need = retention_msr_epilogue_workspace_size(B, H, 1, dv, d_out, dtype);
    if (need == 0) return RET_ERR_UNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < need) return RET_ERR_WORKSPACE;
    if (ret::recurrent_step_tiles(B, H, dv) != 1) {  // rows split over workgroups: the general output stage
        s = retention_recurrent_step(q, k, v, o, state, B, H, dk, dv, dtype, gamma, theta, pos, stream);
        if (s != RET_OK) return s;
        return retention_msr_epilogue(o, gate, gn_weight, gn_bias, eps, w_o, y, B, H, 1, dv, d_out, dtype,
                                      workspace, workspace_bytes, stream);
    }
    // each workgroup of the step owns a whole (sequence, head) row: it also writes the
    // normalised, gated row into the workspace, and only the projection follows
    hipStream_t st = static_cast<hipStream_t>(stream);
    ret::StepArgs a = step_args(q, k, v, o, state, pos, B, H, dk, dv, dtype);
    a.gate = static_cast<const ret::u16*>(gate);
    a.gn_w = gn_weight;
    a.gn_b = gn_bias;
    a.z = static_cast<ret::u16*>(workspace);
    a.eps = eps;
    if (ret::launch_recurrent_step(a, hp, st) != hipSuccess) return RET_ERR_HIP;
    return msr_projection(w_o, y, B, H, 1, dv, d_out, workspace, st);
}

size_t retention_parallel_workspace_size(int B, int H, int N, int dk, int dv, ret_dtype_t dtype) {
    if (B < 1 || H < 1 || N < 1 || dk < 1 || dv < 1 || dtype != RET_BF16 || H > RETENTION_MAX_HEADS) return 0;
    if (!ret::parallel_wide_supported(dk, dv, false)) return 0;
    if (static_cast<long long>(N) * B * H > 2147483647LL) return 0;
    return ret::parallel_wide_workspace(B, H, N, dv);
}

ret_status_t retention_parallel_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                                    int dk, int dv, ret_dtype_t dtype, const float* gamma, const float* theta,
                                    int64_t pos0, void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !o) return RET_ERR_NULL;
    ret_status_t s = check_common(B, H, N, dk, dv, dtype, theta);
    if (s != RET_OK) return s;
    HeadParams hp;
    s = fill_head_params(hp, H, dk, gamma, theta);
    if (s != RET_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace))
        return RET_ERR_ALIGN;
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
    a.split_t = 0;
    a.part = nullptr;
    a.ctr = nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == RET_BF16 && ret::parallel_wide_supported(dk, dv, theta != nullptr)) {
        a.nvt = dv / 128;  // the single-wave-per-SIMD kernel's 128-column value tiles
        const size_t need = ret::parallel_wide_workspace(B, H, N, dv);
        if (workspace && need > 0) {  // the balanced schedule; without a workspace every walk runs whole
            if (workspace_bytes < need) return RET_ERR_WORKSPACE;
            ret::parallel_wide_bind(a, workspace);
        }
        return ret::launch_parallel_wide(a, hp, st) == hipSuccess ? RET_OK : RET_ERR_HIP;
    }
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

    const ret::StepArgs a = step_args(q, k, v, o, state, pos, B, H, dk, dv, dtype);
    const hipError_t e = ret::launch_recurrent_step(a, hp, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RET_OK : RET_ERR_HIP;
}

}  // extern "C"
