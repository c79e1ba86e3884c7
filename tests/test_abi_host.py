"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/retention.h declares,
and reject bad arguments with the documented status codes before any HIP
call: every call here fails validation, so nothing reaches the GPU.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "retention.h")
PKG = os.path.join(ROOT, "linear_attention_sequence_fwd_amd")

OK, NULL, SHAPE, DTYPE, GAMMA, UNSUP, WS, ALIGN = 0, 1, 2, 3, 4, 5, 6, 7
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    import linear_attention_sequence_fwd_amd as ret

    if not os.path.exists(ret.LIB_PATH):
        from linear_attention_sequence_fwd_amd import build

        build.build(verbose=False)
    return ret.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(retention_\w+)\s*\(", text, re.M)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("retention_parallel_fwd", "retention_chunkwise_fwd", "retention_recurrent_step",
              "retention_chunkwise_workspace_size", "retention_status_string", "retention_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.retention_abi_version() == 4
    for s in range(9):
        assert len(lib.retention_status_string(s)) > 0
    assert lib.retention_status_string(123) == b"unknown status"


A = 0x10000  # fake, 16-byte aligned device address: validation never dereferences it


def chunk(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, B=1, H=2, N=100, dk=64, dv=64, dtype=BF16, chunk=64, gamma=None,
             theta=None, pos0=0, state_in=None, state_out=None, segments=0, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.retention_chunkwise_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["N"], a["dk"],
                                       a["dv"], a["dtype"], a["chunk"], a["gamma"], a["theta"], a["pos0"],
                                       a["state_in"], a["state_out"], a["segments"], a["ws"], a["ws_bytes"],
                                       None)


def par(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, B=1, H=2, N=100, dk=64, dv=64, dtype=BF16, gamma=None, theta=None, pos0=0,
             ws=None, ws_bytes=0)
    a.update(kw)
    return lib.retention_parallel_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["N"], a["dk"], a["dv"],
                                      a["dtype"], a["gamma"], a["theta"], a["pos0"], a["ws"], a["ws_bytes"], None)


def step(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, state=A, B=1, H=2, dk=64, dv=64, dtype=BF16, gamma=None, theta=None, pos=None)
    a.update(kw)
    return lib.retention_recurrent_step(a["q"], a["k"], a["v"], a["o"], a["state"], a["B"], a["H"], a["dk"],
                                        a["dv"], a["dtype"], a["gamma"], a["theta"], a["pos"], None)


def floats(*x):
    arr = (ctypes.c_float * len(x))(*x)
    return ctypes.cast(arr, ctypes.c_void_p), arr


def test_null_pointers(lib):
    for key in ("q", "k", "v", "o"):
        assert chunk(lib, **{key: None}) == NULL
        assert par(lib, **{key: None}) == NULL
        assert step(lib, **{key: None}) == NULL
    assert step(lib, state=None) == NULL
    th, _keep = floats(*([1.0] * 32))
    assert step(lib, theta=th, pos=None) == NULL


def test_bad_shapes_and_dtype(lib):
    for key in ("B", "H", "N", "dk", "dv"):
        assert chunk(lib, **{key: 0}) == SHAPE
        assert par(lib, **{key: -1}) == SHAPE
    assert chunk(lib, dtype=7) == DTYPE
    assert step(lib, dtype=-1) == DTYPE
    th, _keep = floats(*([1.0] * 32))
    assert chunk(lib, dk=63, theta=th, dtype=F32) == SHAPE
    assert chunk(lib, segments=-1) == SHAPE


def test_gamma_and_theta_validation(lib):
    for bad in (0.0, -0.5, 1.5, float("nan"), float("inf")):
        g, _keep = floats(0.9, bad)
        assert chunk(lib, gamma=g) == GAMMA
        assert par(lib, gamma=g) == GAMMA
        assert step(lib, gamma=g) == GAMMA
    th, _keep = floats(*([1.0] * 31 + [float("nan")]))
    assert chunk(lib, theta=th) == GAMMA


def test_unsupported_sets(lib):
    assert chunk(lib, chunk=48) == UNSUP  # chunks: 16, 32, 64, 128 and (bf16) multiples of 128
    assert chunk(lib, chunk=8) == UNSUP
    assert chunk(lib, chunk=48) == UNSUP
    assert chunk(lib, chunk=100) == UNSUP
    assert chunk(lib, dk=96) == UNSUP          # bf16 dk outside {64,128,256}
    assert chunk(lib, dv=96) == UNSUP          # bf16 dv not a multiple of 64
    assert chunk(lib, dtype=F32, dk=256, chunk=64) == UNSUP  # f32 chunk*dk > 8192
    assert chunk(lib, H=129) == UNSUP
    th, _keep = floats(*([1.0] * 256))
    assert chunk(lib, dk=512, theta=th, dtype=F32) == UNSUP
    assert par(lib, dtype=F32, dk=256) == UNSUP
    assert step(lib, dv=1028) == UNSUP
    assert step(lib, dv=6) == UNSUP


def test_alignment(lib):
    assert chunk(lib, q=A + 2) == ALIGN
    assert chunk(lib, state_in=A + 4) == ALIGN
    assert par(lib, o=A + 8) == ALIGN
    assert step(lib, state=A + 4) == ALIGN


def test_workspace_contract(lib):
    # few heads: the library splits the sequence and needs a workspace
    need = lib.retention_chunkwise_workspace_size(1, 2, 4096, 64, 64, BF16, 64, 0)
    assert need > 0
    assert chunk(lib, N=4096, ws=None, ws_bytes=0) == WS
    assert chunk(lib, N=4096, ws=A, ws_bytes=need - 1) == WS
    # invalid sizes report 0
    assert lib.retention_chunkwise_workspace_size(1, 2, 4096, 64, 64, BF16, 33, 0) == 0
    assert lib.retention_chunkwise_workspace_size(0, 2, 4096, 64, 64, BF16, 64, 0) == 0
    # many heads: no split, no workspace
    assert lib.retention_chunkwise_workspace_size(4, 16, 8192, 256, 512, BF16, 128, 0) == 0
    # requested segments are honoured up to 512 (batch x heads x value tiles) chains, ignored beyond
    assert lib.retention_chunkwise_workspace_size(4, 128, 4096, 64, 64, BF16, 64, 4) > 0
    assert lib.retention_chunkwise_workspace_size(5, 128, 4096, 64, 64, BF16, 64, 4) == 0


def test_parallel_workspace_contract(lib):
    """The parallel form asks for a workspace only where it splits long causal walks: bf16 without
    rotation at d_k 64 / 128, d_v a multiple of 128, at most 512 query blocks of 128 over heads
    and value tiles. 4096 tokens, 8 heads of 128: 32 blocks a head, walks longer than 16 split,
    so 16 x 8 split blocks, each with two 128 x 128 float32 partials, after a fixed region of 256
    tickets (at most 512 blocks, at most half of them split)."""
    need = lib.retention_parallel_workspace_size(1, 8, 4096, 128, 128, BF16)
    assert need == 1024 + 16 * 8 * 2 * 128 * 128 * 4  # 256 tickets first, whatever the sizes
    assert lib.retention_parallel_workspace_size(1, 8, 4096, 64, 256, BF16) == 1024 + 16 * 16 * 2 * 128 * 128 * 4
    assert lib.retention_parallel_workspace_size(1, 8, 4096, 128, 128, F32) == 0      # the f32 kernel
    assert lib.retention_parallel_workspace_size(1, 8, 4096, 256, 128, BF16) == 0     # d_k 256: another kernel
    assert lib.retention_parallel_workspace_size(1, 8, 4096, 128, 64, BF16) == 0      # d_v 64: another kernel
    assert lib.retention_parallel_workspace_size(1, 8, 128, 128, 128, BF16) == 0      # one query block a head
    assert lib.retention_parallel_workspace_size(4, 16, 4096, 128, 128, BF16) == 0    # 2048 blocks: no split
    assert lib.retention_parallel_workspace_size(1, 16, 4096, 128, 128, BF16) > 0     # 512 blocks: split
    assert lib.retention_parallel_workspace_size(0, 8, 4096, 128, 128, BF16) == 0
    # a workspace, when given, must be large enough and aligned; none is also valid (whole walks)
    assert par(lib, H=8, N=4096, dk=128, dv=128, ws=A, ws_bytes=need - 1) == WS
    assert par(lib, H=8, N=4096, dk=128, dv=128, ws=A + 8, ws_bytes=need) == ALIGN


@pytest.mark.parametrize("cfg", [(1, 8, 64, 64, BF16, 64), (1, 8, 128, 128, BF16, 128), (2, 8, 64, 64, F32, 64),
                                 (1, 1, 64, 64, F32, 64)])
def test_workspace_does_not_depend_on_length(lib, cfg):
    """The resident state of the method does not grow with context ("Retentive
    Networks (RetNet)" implementer checklist); neither does this workspace."""
    B, H, dk, dv, dt, C = cfg
    sizes = {lib.retention_chunkwise_workspace_size(B, H, N, dk, dv, dt, C, 0) for N in (1024, 8192, 65536, 1 << 20)}
    assert len(sizes) == 1


def test_product_path_never_touches_the_oracle():
    imp = re.compile(r"^\s*(from\s+oracle\b|import\s+oracle\b|from\s+\.+oracle\b)", re.M)
    inc = re.compile(r'#\s*include\s*[<"][^>"]*oracle', re.M)
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            path = os.path.join(dirpath, f)
            if f.endswith(".py"):
                assert not imp.search(open(path).read()), path
            elif f.endswith((".hip", ".hpp", ".cpp", ".h")):
                assert not inc.search(open(path).read()), path


def bwd(lib, **kw):
    a = dict(q=A, k=A, v=A, d_o=A, d_q=A, d_k=A, d_v=A, B=1, H=2, N=100, dk=64, dv=64, dtype=BF16, chunk=64,
             gamma=None, theta=None, pos0=0, state_in=None, d_state_out=None, d_state_in=None, ws=None,
             ws_bytes=0)
    a.update(kw)
    return lib.retention_chunkwise_bwd(a["q"], a["k"], a["v"], a["d_o"], a["d_q"], a["d_k"], a["d_v"], a["B"],
                                       a["H"], a["N"], a["dk"], a["dv"], a["dtype"], a["chunk"], a["gamma"],
                                       a["theta"], a["pos0"], a["state_in"], a["d_state_out"], a["d_state_in"],
                                       a["ws"], a["ws_bytes"], None)


def test_backward_validation(lib):
    for key in ("q", "k", "v", "d_o", "d_q", "d_k", "d_v"):
        assert bwd(lib, **{key: None}) == NULL
    for key in ("B", "H", "N", "dk", "dv"):
        assert bwd(lib, **{key: 0}) == SHAPE
    assert bwd(lib, dtype=5) == DTYPE
    g, _keep = floats(0.9, 1.5)
    assert bwd(lib, gamma=g) == GAMMA
    assert bwd(lib, d_state_in=A + 4) == ALIGN
    assert bwd(lib, d_o=A + 2) == ALIGN
    # each of dk and dv is the key width of some pass: dk must be a bf16 key width, and dv one or twice one
    # (a dv of 512 runs the first two passes over its halves)
    assert bwd(lib, dv=512) == WS
    assert bwd(lib, dk=256, dv=512, chunk=128) == WS
    assert bwd(lib, dv=1024) == UNSUP
    assert bwd(lib, dk=512, dv=64) == UNSUP
    assert bwd(lib, chunk=48) == UNSUP
    assert bwd(lib, dtype=F32, dk=64, dv=200) == UNSUP  # not a multiple of 8 / 16
    # the state gradient divides by gamma: tiny gammas are outside the set only then
    tiny, _keep2 = floats(0.9, 1e-7)
    need = lib.retention_chunkwise_bwd_workspace_size(1, 2, 100, 64, 64, BF16, 64)
    assert bwd(lib, gamma=tiny, d_state_out=A, ws=A, ws_bytes=need) == UNSUP
    # the workspace is always needed (reversed copies of the inputs) and grows with N
    assert need > 0
    assert bwd(lib) == WS
    assert bwd(lib, ws=A, ws_bytes=need - 1) == WS
    assert lib.retention_chunkwise_bwd_workspace_size(1, 2, 200, 64, 64, BF16, 64) > need
    assert lib.retention_chunkwise_bwd_workspace_size(1, 2, 100, 64, 512, BF16, 64) > 0
    assert lib.retention_chunkwise_bwd_workspace_size(1, 2, 100, 64, 1024, BF16, 64) == 0
    assert lib.retention_chunkwise_bwd_workspace_size(1, 2, 100, 64, 64, BF16, 48) == 0


def epi(lib, **kw):
    a = dict(o=A, gate=None, w=None, b=None, eps=1e-6, w_o=A, y=A, B=1, H=2, N=100, dv=64, d_out=128, dtype=BF16,
             ws=None, ws_bytes=0)
    a.update(kw)
    return lib.retention_msr_epilogue(a["o"], a["gate"], a["w"], a["b"], a["eps"], a["w_o"], a["y"], a["B"], a["H"],
                                      a["N"], a["dv"], a["d_out"], a["dtype"], a["ws"], a["ws_bytes"], None)


def test_epilogue_validation(lib):
    for key in ("o", "w_o", "y"):
        assert epi(lib, **{key: None}) == NULL
    for key in ("B", "H", "N", "dv", "d_out"):
        assert epi(lib, **{key: 0}) == SHAPE
    assert epi(lib, dtype=9) == DTYPE
    assert epi(lib, eps=-1.0) == GAMMA
    assert epi(lib, eps=float("nan")) == GAMMA
    assert epi(lib, gate=A + 2) == ALIGN
    assert epi(lib, dtype=F32) == UNSUP
    assert epi(lib, dv=96) == UNSUP
    assert epi(lib, d_out=100) == UNSUP
    need = lib.retention_msr_epilogue_workspace_size(1, 2, 100, 64, 128, BF16)
    assert need >= 100 * 128 * 2
    assert epi(lib) == WS
    assert epi(lib, ws=A, ws_bytes=need - 1) == WS
    assert lib.retention_msr_epilogue_workspace_size(1, 2, 100, 64, 100, BF16) == 0


def test_decode_msr_validation(lib):
    def call(**kw):
        a = dict(q=A, k=A, v=A, state=A, B=2, H=2, dk=64, dv=64, dtype=BF16, gamma=None, theta=None, pos=None,
                 gate=None, w=None, b=None, eps=1e-6, w_o=A, d_out=128, o=A, y=A, ws=None, ws_bytes=0)
        a.update(kw)
        return lib.retention_recurrent_step_msr(a["q"], a["k"], a["v"], a["state"], a["B"], a["H"], a["dk"], a["dv"],
                                                a["dtype"], a["gamma"], a["theta"], a["pos"], a["gate"], a["w"], a["b"],
                                                a["eps"], a["w_o"], a["d_out"], a["o"], a["y"], a["ws"], a["ws_bytes"],
                                                None)
    for key in ("q", "k", "v", "state", "w_o", "o", "y"):
        assert call(**{key: None}) == NULL
    assert call(B=0) == SHAPE
    assert call(d_out=0) == SHAPE
    assert call(dtype=4) == DTYPE
    assert call(eps=-1.0) == GAMMA
    assert call(y=A + 2) == ALIGN
    assert call(dtype=F32) == UNSUP
    assert call(d_out=100) == UNSUP
    assert call() == WS


def test_large_chunks(lib):
    assert chunk(lib, chunk=192) == UNSUP              # not a multiple of 128
    assert chunk(lib, chunk=256, dtype=F32) == UNSUP   # large chunks are bf16 only
    assert chunk(lib, chunk=1 << 17) == UNSUP
    # one state per chunk: the workspace grows with N / chunk
    w1 = lib.retention_chunkwise_workspace_size(1, 2, 4096, 64, 64, BF16, 512, 0)
    w2 = lib.retention_chunkwise_workspace_size(1, 2, 16384, 64, 64, BF16, 512, 0)
    assert 0 < w1 < w2
    assert chunk(lib, N=4096, chunk=512, ws=A, ws_bytes=w1 - 1) == WS
    # more than 4096 chunks per sequence is outside the set
    assert lib.retention_chunkwise_workspace_size(1, 1, 4097 * 256, 64, 64, BF16, 256, 0) == 0


def test_large_chunk_workspace_holds_every_chunk(lib):
    # 65536 tokens in chunks of 256 are 256 segments per chain: the workspace
    # must hold one 128 x 128 float32 state per segment for each of the 8
    # chains (a plan that capped the count at the automatic limit of 64 sized
    # it for a quarter of them while the kernel indexed all 256)
    need = lib.retention_chunkwise_workspace_size(1, 8, 65536, 128, 128, BF16, 256, 0)
    assert need >= 8 * 256 * 128 * 128 * 4
    assert need > lib.retention_chunkwise_workspace_size(1, 8, 16384, 128, 128, BF16, 256, 0)


def test_small_chunks(lib):
    # 16- and 32-token chunks in both dtypes; bf16 runs a 16-token chunk as 32-token tiles
    for dt in (F32, BF16):
        assert lib.retention_chunkwise_workspace_size(1, 2, 4096, 64, 64, dt, 16, 0) > 0
        assert lib.retention_chunkwise_workspace_size(1, 2, 4096, 64, 64, dt, 32, 0) > 0
    st, p = plan(lib, 1, 2, 4096, 64, 64, BF16, 16, 0)
    assert st == OK and p.tile == 32
    st, p = plan(lib, 1, 2, 4096, 64, 64, F32, 16, 0)
    assert st == OK and p.tile == 16


# ------------------------------------------------------------ workspace plans


class Plan(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int), ("dv_tile", ctypes.c_int), ("value_tiles", ctypes.c_int),
                ("segments", ctypes.c_int), ("segment_len", ctypes.c_int), ("group_len", ctypes.c_int),
                ("segments_max", ctypes.c_int), ("reserved", ctypes.c_int),
                ("flags_off", ctypes.c_uint64), ("gflags_off", ctypes.c_uint64), ("agg_off", ctypes.c_uint64),
                ("gagg_off", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64)]


CTL_STRIDE = FLAG_STRIDE = 16 * 8  # bytes between two counters / two flags (one 128-byte line each)


def plan(lib, B, H, N, dk, dv, dtype, chunk, segments):
    p = Plan()
    st = lib.retention_chunkwise_plan(B, H, N, dk, dv, dtype, chunk, segments, ctypes.byref(p))
    return st, p


def plan_grid():
    for dtype in (F32, BF16):
        for B, H in ((1, 1), (1, 8), (2, 3), (4, 16), (64, 16)):
            for N in (1, 63, 128, 1000, 2048, 65536, 200000):
                for dk, dv in ((64, 64), (128, 128), (256, 128), (256, 512), (64, 192)):
                    for chunk in (16, 32, 64, 128, 256, 1024, 8192):
                        for segments in (0, 1, 3, 64, 300):
                            yield dtype, B, H, N, dk, dv, chunk, segments


def test_every_plan_indexes_inside_its_workspace(lib):
    """Every offset the segmented kernels form lies inside the workspace the
    call requires: ticket counters, segment and group flags, published
    segment states and group aggregates (the fault class of a plan whose
    workspace held fewer segments than its kernel indexed)."""
    checked = 0
    for dtype, B, H, N, dk, dv, C, seg in plan_grid():
        st, p = plan(lib, B, H, N, dk, dv, dtype, C, seg)
        size = lib.retention_chunkwise_workspace_size(B, H, N, dk, dv, dtype, C, seg)
        if st != OK:
            assert st in (SHAPE, UNSUP) and size == 0, (dtype, B, H, N, dk, dv, C, seg, st)
            continue
        checked += 1
        case = (dtype, B, H, N, dk, dv, C, seg)
        assert size == p.workspace_bytes, case
        assert p.value_tiles * p.dv_tile == dv and p.segment_len % p.tile == 0, case
        assert p.segments == -(-N // p.segment_len), case  # every token belongs to a segment
        assert (p.segments - 1) * p.segment_len < N, case   # no empty segment
        assert 1 <= p.segments <= p.segments_max, case
        if p.segments == 1:
            continue
        chains = B * H * p.value_tiles
        groups = -(-p.segments // p.group_len)
        assert p.workspace_bytes > 0, case
        assert 0 < p.flags_off <= p.gflags_off <= p.agg_off <= p.gagg_off <= p.workspace_bytes, case
        # one 8-byte ticket counter per chain at chain * 128 bytes
        assert (chains - 1) * CTL_STRIDE + 8 <= p.flags_off, case
        if dtype == BF16:
            assert p.flags_off + ((chains - 1) * p.segments + p.segments - 1) * FLAG_STRIDE + 8 <= p.gflags_off, case
            assert p.gflags_off + ((chains - 1) * groups + groups - 1) * FLAG_STRIDE + 8 <= p.agg_off, case
            slot = dk * p.dv_tile * 4
            assert p.agg_off + chains * p.segments * slot <= p.gagg_off, case
            assert p.gagg_off + chains * groups * slot <= p.workspace_bytes, case
            if dk in (128, 256) and p.dv_tile == 128 and p.tile == 128:
                # the wide kernel's three-kernel form (unrotated calls): [B, H, segments, dk, dv]
                assert p.agg_off + B * H * p.segments * dk * dv * 4 <= p.gagg_off, case
        else:  # float32 pre-pass and scan: [B, H, segments, dk, dv]
            assert p.agg_off + B * H * p.segments * dk * dv * 4 <= p.gagg_off, case
    assert checked > 1000
