"""MI355X-native multi-scale retention: Python binding of the C ABI.

The functions below share the names of the C entry points declared in
include/retention.h and only marshal arguments: torch tensors supply device
memory and the current HIP stream, every step of retention runs in the HIP
kernels of libretention_mi355x.so. There is no CPU or PyTorch fallback: if
the library is missing, importing a function raises.
"""

import ctypes
import os

__all__ = [
    "RetentionError",
    "HostFloats",
    "load_library",
    "retention_parallel_fwd",
    "retention_parallel_workspace_size",
    "retention_chunkwise_fwd",
    "retention_chunkwise_fwd_timed",
    "retention_chunkwise_workspace_size",
    "retention_recurrent_step",
    "retention_chunkwise_bwd",
    "retention_chunkwise_bwd_workspace_size",
    "retention_msr_epilogue",
    "retention_msr_epilogue_workspace_size",
    "retention_recurrent_step_msr",
    "retention_status_string",
    "retention_abi_version",
    "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libretention_mi355x.so")

RET_F32 = 0
RET_BF16 = 1

_STATUS = {
    0: "RET_OK",
    1: "RET_ERR_NULL",
    2: "RET_ERR_SHAPE",
    3: "RET_ERR_DTYPE",
    4: "RET_ERR_GAMMA",
    5: "RET_ERR_UNSUPPORTED",
    6: "RET_ERR_WORKSPACE",
    7: "RET_ERR_ALIGN",
    8: "RET_ERR_HIP",
}

_lib = None


class RetentionError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        self.code = _STATUS.get(status, str(status))
        super().__init__(f"{what}: {self.code} ({retention_status_string(status)})")


def load_library(path=None):
    """Load (once) and return the ctypes handle of the HIP library."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m linear_attention_sequence_fwd_amd.build`"
        )
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.retention_parallel_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, fp, fp, i64, vp, sz, vp]
    lib.retention_parallel_fwd.restype = i32
    lib.retention_parallel_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.retention_parallel_workspace_size.restype = sz
    lib.retention_chunkwise_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, fp, fp, i64,
                                            vp, vp, i32, vp, sz, vp]
    lib.retention_chunkwise_fwd.restype = i32
    lib.retention_chunkwise_fwd_timed.argtypes = lib.retention_chunkwise_fwd.argtypes + [vp]
    lib.retention_chunkwise_fwd_timed.restype = i32
    lib.retention_chunkwise_fwd_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, fp, fp,
                                                    i64, vp, vp, i32, vp]
    lib.retention_chunkwise_fwd_noalloc.restype = i32
    lib.retention_chunkwise_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    lib.retention_chunkwise_workspace_size.restype = sz
    lib.retention_recurrent_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, fp, fp, vp, vp]
    lib.retention_recurrent_step.restype = i32
    lib.retention_chunkwise_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, fp,
                                            fp, i64, vp, vp, vp, vp, sz, vp]
    lib.retention_chunkwise_bwd.restype = i32
    lib.retention_chunkwise_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.retention_chunkwise_bwd_workspace_size.restype = sz
    f32 = ctypes.c_float
    lib.retention_msr_epilogue.argtypes = [vp, vp, vp, vp, f32, vp, vp, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.retention_msr_epilogue.restype = i32
    lib.retention_msr_epilogue_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.retention_msr_epilogue_workspace_size.restype = sz
    lib.retention_recurrent_step_msr.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, fp, fp, vp, vp, vp, vp,
                                                 f32, vp, i32, vp, vp, vp, sz, vp]
    lib.retention_recurrent_step_msr.restype = i32
    lib.retention_status_string.argtypes = [i32]
    lib.retention_status_string.restype = ctypes.c_char_p
    lib.retention_abi_version.argtypes = []
    lib.retention_abi_version.restype = i32
    _lib = lib
    return lib


def retention_status_string(status):
    return load_library().retention_status_string(int(status)).decode()


def retention_abi_version():
    return int(load_library().retention_abi_version())


# ---------------------------------------------------------------- marshalling


def _torch():
    import torch

    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RET_BF16
    if t.dtype == torch.float32:
        return RET_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("retention tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("retention tensors must be contiguous")


class HostFloats:
    """A host float array marshalled once for repeated calls (gamma or theta).

    Passing one of these instead of a list or tensor skips the per-call
    conversion, which matters for launch-bound callers."""

    def __init__(self, vals):
        torch = _torch()
        if isinstance(vals, torch.Tensor):
            vals = vals.detach().to("cpu", torch.float32).tolist()
        self.values = [float(x) for x in vals]
        self.array = (ctypes.c_float * len(self.values))(*self.values)
        self.pointer = ctypes.cast(self.array, ctypes.c_void_p)

    def __len__(self):
        return len(self.values)


def _host_floats(vals, n, what):
    if vals is None:
        return None, None
    if not isinstance(vals, HostFloats):
        vals = HostFloats(vals)
    if len(vals) != n:
        raise ValueError(f"{what} needs {n} values, got {len(vals)}")
    return vals, vals.pointer


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _raise(status, what):
    if status != 0:
        raise RetentionError(status, what)


def retention_parallel_workspace_size(B, H, N, dk, dv, dtype):
    torch = _torch()
    code = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    return int(load_library().retention_parallel_workspace_size(B, H, N, dk, dv, code))


def retention_parallel_fwd(q, k, v, gamma=None, theta=None, pos0=0, out=None, workspace=None, balanced=True,
                           stream=None):
    """O = ((Q K^T) (.) D) V for q, k [B,H,N,dk] and v [B,H,N,dv] (bf16 or fp32).

    With balanced (the default) and no workspace given, a cached zero-filled
    workspace lets the library split the longest causal walks over two
    workgroups; balanced=False runs every query block's walk whole."""
    torch = _torch()
    _check_dev(q, k, v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=v.dtype, device=v.device)
    _check_dev(out)
    if workspace is None and balanced:
        nbytes = retention_parallel_workspace_size(B, H, N, dk, dv, q.dtype)
        if nbytes:
            workspace = _cached_workspace(nbytes, v.device, stream, kind="parallel")
    _g, g = _host_floats(gamma, H, "gamma")
    _t, th = _host_floats(theta, dk // 2, "theta")
    st = load_library().retention_parallel_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, dk, dv, _dtype_code(q), g, th, int(pos0), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream)
    )
    _raise(st, "retention_parallel_fwd")
    return out


_WORKSPACES = {}


def _cached_workspace(nbytes, device, stream, kind="fwd"):
    """Zero-filled workspace of at least nbytes for calls on `stream` (the
    current stream when None). Growing it allocates and zero-fills a new
    buffer, ordered on that stream before the call that uses it. Forward and
    backward calls keep separate buffers (`kind`): the backward's scratch must
    not land on a forward call's counters."""
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (kind, device.index if device.index is not None else torch.cuda.current_device(), s.cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def retention_chunkwise_workspace_size(B, H, N, dk, dv, dtype, chunk, segments=0):
    torch = _torch()
    code = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    return int(load_library().retention_chunkwise_workspace_size(B, H, N, dk, dv, code, chunk, segments))


def retention_chunkwise_fwd(q, k, v, chunk=64, gamma=None, theta=None, pos0=0, state_in=None,
                            return_state=False, state_out=None, segments=0, out=None, workspace=None,
                            stream=None, events=None):
    """Chunkwise retention forward. Returns o, or (o, state) with return_state.

    state_in / state_out are float32 [B,H,dk,dv] device tensors (state_out may
    be state_in). Without `workspace` the call uses a zero-filled workspace
    this module keeps per (device, stream) and grows as needed; a caller's own
    workspace must be zero-filled before its first use (the library leaves it
    ready for the next call). With `events` (six torch.cuda.Event created
    with enable_timing=True: start/stop of the segment pre-pass, the segment
    scan and the main kernel) the call goes through
    retention_chunkwise_fwd_timed.
    """
    torch = _torch()
    _check_dev(q, k, v, state_in, state_out)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=v.dtype, device=v.device)
    if return_state and state_out is None:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=v.device)
    _check_dev(out)
    ws_bytes = retention_chunkwise_workspace_size(B, H, N, dk, dv, q.dtype, chunk, segments)
    if ws_bytes and workspace is None:
        workspace = _cached_workspace(ws_bytes, v.device, stream)
    _g, g = _host_floats(gamma, H, "gamma")
    _t, th = _host_floats(theta, dk // 2, "theta")
    args = [
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, dk, dv, _dtype_code(q), int(chunk), g, th, int(pos0),
        _ptr(state_in), _ptr(state_out), int(segments), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream),
    ]
    lib = load_library()
    if events is None:
        st = lib.retention_chunkwise_fwd(*args)
        _raise(st, "retention_chunkwise_fwd")
    else:
        if len(events) != 6:
            raise ValueError("events needs six torch.cuda.Event")
        for e in events:
            e.record()  # materialise the underlying hipEvent_t
        evs = (ctypes.c_void_p * 6)(*[e.cuda_event for e in events])
        st = lib.retention_chunkwise_fwd_timed(*args, ctypes.cast(evs, ctypes.c_void_p))
        _raise(st, "retention_chunkwise_fwd_timed")
    return (out, state_out) if return_state else out


def retention_chunkwise_fwd_noalloc(q, k, v, out, chunk=64, gamma=None, theta=None, pos0=0, state_in=None,
                                    state_out=None, segments=0, stream=None):
    """retention_chunkwise_fwd without a workspace (the library's device array
    serves instead; calls on one GPU must not overlap). `out` (and state_out,
    when wanted) are the caller's device tensors."""
    _check_dev(q, k, v, out, state_in, state_out)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    _g, g = _host_floats(gamma, H, "gamma")
    _t, th = _host_floats(theta, dk // 2, "theta")
    st = load_library().retention_chunkwise_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, dk, dv, _dtype_code(q), int(chunk), g, th, int(pos0),
        _ptr(state_in), _ptr(state_out), int(segments), _stream(stream))
    _raise(st, "retention_chunkwise_fwd_noalloc")
    return out


def retention_chunkwise_fwd_timed(q, k, v, events, **kw):
    """retention_chunkwise_fwd recording the six phase events (see the C header)."""
    return retention_chunkwise_fwd(q, k, v, events=events, **kw)


def retention_chunkwise_bwd_workspace_size(B, H, N, dk, dv, dtype, chunk):
    torch = _torch()
    code = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    return int(load_library().retention_chunkwise_bwd_workspace_size(B, H, N, dk, dv, code, chunk))


def retention_chunkwise_bwd(q, k, v, d_o, chunk=64, gamma=None, theta=None, pos0=0, state_in=None,
                            d_state_out=None, need_d_state_in=False, d_state_in=None, out=None,
                            workspace=None, stream=None):
    """Gradients of retention_chunkwise_fwd: returns (d_q, d_k, d_v, d_state_in).

    d_o has the shape and dtype of the forward's output; d_state_out (float32
    [B,H,dk,dv] or None) is the gradient of its final state. d_state_in is
    returned (float32 [B,H,dk,dv]) when need_d_state_in or a d_state_in tensor
    is given, else None. `out` may supply (d_q, d_k, d_v). Without `workspace`
    the call uses a per-stream workspace this module keeps for backward calls.
    """
    torch = _torch()
    _check_dev(q, k, v, d_o, state_in, d_state_out, d_state_in)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    d_q, d_k, d_v = out
    _check_dev(d_q, d_k, d_v)
    if need_d_state_in and d_state_in is None:
        d_state_in = torch.empty((B, H, dk, dv), dtype=torch.float32, device=v.device)
    ws_bytes = retention_chunkwise_bwd_workspace_size(B, H, N, dk, dv, q.dtype, chunk)
    if workspace is None and ws_bytes:
        workspace = _cached_workspace(ws_bytes, v.device, stream, kind="bwd")
    _g, g = _host_floats(gamma, H, "gamma")
    _t, th = _host_floats(theta, dk // 2, "theta")
    st = load_library().retention_chunkwise_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(d_o), _ptr(d_q), _ptr(d_k), _ptr(d_v), B, H, N, dk, dv, _dtype_code(q),
        int(chunk), g, th, int(pos0), _ptr(state_in), _ptr(d_state_out), _ptr(d_state_in), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream),
    )
    _raise(st, "retention_chunkwise_bwd")
    return d_q, d_k, d_v, d_state_in


def retention_msr_epilogue_workspace_size(B, H, N, dv, d_out, dtype):
    torch = _torch()
    code = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    return int(load_library().retention_msr_epilogue_workspace_size(B, H, N, dv, d_out, code))


def retention_msr_epilogue(o, w_o, gn_weight=None, gn_bias=None, gate=None, eps=1e-6, out=None, workspace=None,
                           stream=None):
    """y = (GroupNorm(concat heads of o) * gate) w_o^T for o [B,H,N,dv] bf16 and
    w_o [d_out, H*dv] bf16; returns y [B,N,d_out] bf16 (see the C header)."""
    torch = _torch()
    _check_dev(o, w_o, gn_weight, gn_bias, gate)
    B, H, N, dv = o.shape
    d_out = w_o.shape[0]
    if out is None:
        out = torch.empty((B, N, d_out), dtype=o.dtype, device=o.device)
    _check_dev(out)
    if workspace is None:
        nbytes = retention_msr_epilogue_workspace_size(B, H, N, dv, d_out, o.dtype)
        if nbytes:
            workspace = _cached_workspace(nbytes, o.device, stream, kind="epilogue")
    st = load_library().retention_msr_epilogue(
        _ptr(o), _ptr(gate), _ptr(gn_weight), _ptr(gn_bias), float(eps), _ptr(w_o), _ptr(out), B, H, N, dv, d_out,
        _dtype_code(o), _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream),
    )
    _raise(st, "retention_msr_epilogue")
    return out


def retention_recurrent_step_msr(q, k, v, state, w_o, gamma=None, theta=None, pos=None, gate=None, gn_weight=None,
                                 gn_bias=None, eps=1e-6, o=None, out=None, workspace=None, stream=None):
    """One decode step and the layer's output stage: returns (y [B,d_out], o [B,H,dv]); the state is updated in place."""
    torch = _torch()
    _check_dev(q, k, v, state, w_o, pos, gate, gn_weight, gn_bias)
    B, H, dk = q.shape
    dv = v.shape[-1]
    d_out = w_o.shape[0]
    if o is None:
        o = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    if out is None:
        out = torch.empty((B, d_out), dtype=v.dtype, device=v.device)
    _check_dev(o, out)
    if pos is not None and pos.dtype != torch.int64:
        raise TypeError("pos must be int64")
    if workspace is None:
        nbytes = retention_msr_epilogue_workspace_size(B, H, 1, dv, d_out, v.dtype)
        if nbytes:
            workspace = _cached_workspace(nbytes, v.device, stream, kind="epilogue")
    _g, g = _host_floats(gamma, H, "gamma")
    _t, th = _host_floats(theta, dk // 2, "theta")
    st = load_library().retention_recurrent_step_msr(
        _ptr(q), _ptr(k), _ptr(v), _ptr(state), B, H, dk, dv, _dtype_code(q), g, th, _ptr(pos), _ptr(gate),
        _ptr(gn_weight), _ptr(gn_bias), float(eps), _ptr(w_o), d_out, _ptr(o), _ptr(out), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream),
    )
    _raise(st, "retention_recurrent_step_msr")
    return out, o


def retention_recurrent_step(q, k, v, state, gamma=None, theta=None, pos=None, out=None, stream=None):
    """One decode step: state <- gamma state + k^T v (in place); returns o = q state.

    q, k [B,H,dk]; v [B,H,dv]; state float32 [B,H,dk,dv]; pos int64 [B] device
    tensor of absolute positions (needed with theta).
    """
    torch = _torch()
    _check_dev(q, k, v, state, pos)
    B, H, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    _check_dev(out)
    if pos is not None and pos.dtype != torch.int64:
        raise TypeError("pos must be int64")
    _g, g = _host_floats(gamma, H, "gamma")
    _t, th = _host_floats(theta, dk // 2, "theta")
    st = load_library().retention_recurrent_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state), B, H, dk, dv, _dtype_code(q), g, th, _ptr(pos),
        _stream(stream),
    )
    _raise(st, "retention_recurrent_step")
    return out
