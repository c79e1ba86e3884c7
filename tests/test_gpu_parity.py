"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Small cases compare every output element and the carried state; they span
several tiles and end in a ragged chunk. The full-size workloads run exactly
as the benchmark launches them and are compared on sampled heads the oracle
recomputes one by one. Tolerances (relative L2, tensor-wide and per head):
1e-5 for float32 inputs, 2e-2 for bf16 inputs with float32 accumulation.
"""

import numpy as np
import pytest
import torch

import linear_attention_sequence_fwd_amd as R
from linear_attention_sequence_fwd_amd import workloads as W
from oracle import retention as orc

from helpers import BF16_TOL, F32_TOL, assert_close, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    R.load_library()
    yield
    torch.cuda.synchronize()


def _inputs(B, H, N, dk, dv, dtype, seed):
    q, k, v = W.make_qkv(B, H, N, dk, dv, dtype, seed, device="cpu")
    return q, k, v


def _gammas_for(H, gamma):
    return orc.head_gammas(H) if gamma is None else np.asarray(gamma, dtype=np.float64)


# ------------------------------------------------------------ single-head fp32 workload


def test_single_head_f32_all_forms():
    w = W.WORKLOADS["single_head_f32"]
    q, k, v, _ = W.make_workload("single_head_f32", device="cpu")
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(1))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_par = R.retention_parallel_fwd(qd, kd, vd)
    o_chk, s_chk = R.retention_chunkwise_fwd(qd, kd, vd, chunk=w["chunk"], return_state=True)
    state = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device=DEV)
    outs = []
    for n in range(w["N"]):
        outs.append(R.retention_recurrent_step(qd[:, :, n].contiguous(), kd[:, :, n].contiguous(),
                                               vd[:, :, n].contiguous(), state))
    o_rec = torch.stack(outs, dim=2)
    torch.cuda.synchronize()
    assert_close(to64(o_par), ref, F32_TOL, "parallel")
    assert_close(to64(o_chk), ref, F32_TOL, "chunkwise")
    assert_close(to64(s_chk), ref_s, F32_TOL, "chunkwise state")
    assert_close(to64(o_rec), ref, F32_TOL, "recurrent")
    assert_close(to64(state), ref_s, F32_TOL, "recurrent state")


# ------------------------------------------------------------ small bf16 chunkwise, many shapes

BF16_CHUNK_CASES = [
    # B, H, N, dk, dv, chunk, rotary, state_in, segments
    (2, 3, 300, 64, 64, 64, False, False, 0),
    (1, 2, 333, 128, 128, 128, True, True, 0),
    (2, 2, 257, 256, 128, 128, False, True, 0),
    (1, 2, 200, 256, 192, 64, True, False, 0),
    (2, 3, 640, 64, 128, 64, True, True, 3),
    (1, 1, 1000, 128, 64, 128, False, True, 4),
    (1, 2, 1, 64, 64, 64, True, True, 0),
    (1, 2, 63, 128, 128, 128, False, False, 0),
    (1, 1, 4100, 64, 64, 64, True, True, 0),
]


@pytest.mark.parametrize("case", BF16_CHUNK_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}C{}rot{}st{}seg{}".format(*c))
def test_chunkwise_bf16_small(case):
    B, H, N, dk, dv, C, rot, st, seg = case
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=N + dk + dv)
    theta = W.rotary_theta(dk) if rot else None
    s0 = torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(7)) * 0.1 if st else None
    pos0 = 17 if rot else 0
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(H),
                               theta=None if theta is None else to64(theta), pos0=pos0,
                               state0=None if s0 is None else to64(s0))
    o, s = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=C, theta=theta, pos0=pos0,
                                     state_in=None if s0 is None else s0.to(DEV), return_state=True,
                                     segments=seg)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, BF16_TOL, "O")
    assert_close(to64(s), ref_s, BF16_TOL, "state")


# ------------------------------------------------------------ small bf16 parallel

BF16_PAR_CASES = [
    (2, 3, 300, 64, 64, False),
    (1, 2, 513, 128, 128, True),
    (1, 2, 260, 256, 128, False),
    (1, 2, 130, 256, 192, True),
    (1, 1, 1, 64, 64, False),
]


@pytest.mark.parametrize("case", BF16_PAR_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}rot{}".format(*c))
def test_parallel_bf16_small(case):
    B, H, N, dk, dv, rot = case
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=3 * N + dk)
    theta = W.rotary_theta(dk) if rot else None
    ref = orc.parallel(to64(q), to64(k), to64(v), orc.head_gammas(H),
                       theta=None if theta is None else to64(theta), pos0=5)
    o = R.retention_parallel_fwd(q.to(DEV), k.to(DEV), v.to(DEV), theta=theta, pos0=5)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, BF16_TOL, "O")


# ------------------------------------------------------------ float32 paths

F32_CASES = [
    # B, H, N, dk, dv, chunk, rotary, state_in
    (2, 2, 150, 16, 48, 64, True, True),
    (1, 3, 300, 64, 64, 128, False, False),
    (1, 2, 129, 128, 16, 64, True, True),
    (2, 1, 77, 32, 128, 128, False, True),
    # widths that are multiples of 4 but not of 16 (the register micro-tiles step four columns)
    (1, 2, 97, 36, 16, 32, True, True),
    (1, 1, 70, 20, 32, 16, False, True),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}C{}rot{}st{}".format(*c))
def test_f32_chunkwise_and_parallel(case):
    B, H, N, dk, dv, C, rot, st = case
    q, k, v = _inputs(B, H, N, dk, dv, torch.float32, seed=N + 11)
    theta = W.rotary_theta(dk) if rot else None
    s0 = torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(3)) * 0.1 if st else None
    th64 = None if theta is None else to64(theta)
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(H), theta=th64, pos0=3,
                               state0=None if s0 is None else to64(s0))
    o, s = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=C, theta=theta, pos0=3,
                                     state_in=None if s0 is None else s0.to(DEV), return_state=True)
    o_seg = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=C, theta=theta, pos0=3,
                                      state_in=None if s0 is None else s0.to(DEV), segments=2)
    ref_p = orc.parallel(to64(q), to64(k), to64(v), orc.head_gammas(H), theta=th64, pos0=3)
    if dk <= 128:
        o_par = R.retention_parallel_fwd(q.to(DEV), k.to(DEV), v.to(DEV), theta=theta, pos0=3)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, F32_TOL, "chunkwise O")
    assert_close(to64(s), ref_s, F32_TOL, "chunkwise state")
    assert_close(to64(o_seg), ref, F32_TOL, "segmented O")
    if dk <= 128:
        assert_close(to64(o_par), ref_p, F32_TOL, "parallel O")


# ------------------------------------------------------------ decode steps


@pytest.mark.parametrize("dtype,rot", [(torch.bfloat16, False), (torch.bfloat16, True), (torch.float32, True)])
def test_recurrent_step_small(dtype, rot):
    B, H, dk, dv, steps = 3, 2, 64, 96, 5
    s0, qs, ks, vs = W.make_decode(B, H, dk, dv, dtype, steps, 0.01, seed=9)
    theta = W.rotary_theta(dk) if rot else None
    pos = torch.tensor([0, 77, 4000], dtype=torch.int64)
    g = orc.head_gammas(H)
    S = to64(s0)
    state = s0.to(DEV)
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    for t in range(steps):
        o_ref, S = orc.decode_step(to64(qs[t]), to64(ks[t]), to64(vs[t]), S, g,
                                   theta=None if theta is None else to64(theta),
                                   pos=(pos + t).numpy() if rot else None)
        o = R.retention_recurrent_step(qs[t].to(DEV), ks[t].to(DEV), vs[t].to(DEV), state, theta=theta,
                                       pos=(pos + t).to(DEV) if rot else None)
        torch.cuda.synchronize()
        assert_close(to64(o), o_ref, tol, f"o step {t}")
    assert_close(to64(state), S, tol, "final state")


# ------------------------------------------------------------ the largest supported shapes

MAX_CHUNK_CASES = [
    # B, H, N, dk, dv, chunk, rotary, state_in, segments
    (1, 128, 100, 64, 64, 64, True, True, 0),      # the head limit; chains split in two segments
    (1, 2, 300, 256, 1024, 128, True, True, 0),    # widest key dim, eight 128-wide value tiles
    (1, 1, 520, 256, 1024, 64, False, True, 0),    # chunk 64: sixteen 64-wide tiles, nine segments
    (2, 128, 65, 128, 128, 128, False, False, 0),  # 256 chains: one segment each
]


@pytest.mark.parametrize("case", MAX_CHUNK_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}C{}rot{}st{}seg{}".format(*c))
def test_chunkwise_bf16_max_shapes(case):
    B, H, N, dk, dv, C, rot, st, seg = case
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=5 * N + dv)
    theta = W.rotary_theta(dk) if rot else None
    s0 = torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(21)) * 0.05 if st else None
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(H),
                               theta=None if theta is None else to64(theta), pos0=9,
                               state0=None if s0 is None else to64(s0))
    o, s = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=C, theta=theta, pos0=9,
                                     state_in=None if s0 is None else s0.to(DEV), return_state=True,
                                     segments=seg)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, BF16_TOL, "O")
    assert_close(to64(s), ref_s, BF16_TOL, "state")


def test_parallel_bf16_max_heads():
    B, H, N, dk, dv = 1, 128, 70, 128, 256
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=71)
    theta = W.rotary_theta(dk)
    ref = orc.parallel(to64(q), to64(k), to64(v), orc.head_gammas(H), theta=to64(theta), pos0=2)
    o = R.retention_parallel_fwd(q.to(DEV), k.to(DEV), v.to(DEV), theta=theta, pos0=2)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, BF16_TOL, "O")


@pytest.mark.parametrize("dtype,B,H,dk,dv,rot", [
    (torch.bfloat16, 2, 128, 256, 128, True),   # head limit with rotary at the widest key dim
    (torch.bfloat16, 1, 1, 4096, 1024, False),  # widest decode state
    (torch.float32, 1, 2, 4096, 1024, False),
])
def test_recurrent_step_max_shapes(dtype, B, H, dk, dv, rot):
    steps = 3
    s0, qs, ks, vs = W.make_decode(B, H, dk, dv, dtype, steps, 0.01, seed=13)
    theta = W.rotary_theta(dk) if rot else None
    pos = torch.arange(B, dtype=torch.int64) * 1000 + 3
    g = orc.head_gammas(H)
    S = to64(s0)
    state = s0.to(DEV)
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    for t in range(steps):
        o_ref, S = orc.decode_step(to64(qs[t]), to64(ks[t]), to64(vs[t]), S, g,
                                   theta=None if theta is None else to64(theta),
                                   pos=(pos + t).numpy() if rot else None)
        o = R.retention_recurrent_step(qs[t].to(DEV), ks[t].to(DEV), vs[t].to(DEV), state, theta=theta,
                                       pos=(pos + t).to(DEV) if rot else None)
        torch.cuda.synchronize()
        assert_close(to64(o), o_ref, tol, f"o step {t}")
    assert_close(to64(state), S, tol, "final state")


@pytest.mark.parametrize("dtype,B,H,dk,dv,rot", [
    (torch.bfloat16, 1, 2, 128, 512, True),    # 2 (sequence, head) pairs: 8 column tiles of 64
    (torch.bfloat16, 3, 5, 256, 256, False),   # 15 pairs: 4 tiles of 64
    (torch.float32, 2, 1, 64, 384, True),      # 384 = 3 x 128: 2 tiles of 192 columns
])
def test_recurrent_step_column_tiles(dtype, B, H, dk, dv, rot):
    """Small batches split each state's columns over several workgroups."""
    steps = 4
    s0, qs, ks, vs = W.make_decode(B, H, dk, dv, dtype, steps, 0.01, seed=dv + B)
    theta = W.rotary_theta(dk) if rot else None
    pos = torch.arange(B, dtype=torch.int64) * 97 + 11
    g = orc.head_gammas(H)
    S = to64(s0)
    state = s0.to(DEV)
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    for t in range(steps):
        o_ref, S = orc.decode_step(to64(qs[t]), to64(ks[t]), to64(vs[t]), S, g,
                                   theta=None if theta is None else to64(theta),
                                   pos=(pos + t).numpy() if rot else None)
        o = R.retention_recurrent_step(qs[t].to(DEV), ks[t].to(DEV), vs[t].to(DEV), state, theta=theta,
                                       pos=(pos + t).to(DEV) if rot else None)
        torch.cuda.synchronize()
        assert_close(to64(o), o_ref, tol, f"o step {t}")
    assert_close(to64(state), S, tol, "final state")


@pytest.mark.parametrize("pos0", [1_000_000_007, 3 * 2**31 + 5])
@pytest.mark.parametrize("B,H,N,dk,dv,C,seg", [
    (2, 2, 200, 64, 64, 64, 0),     # 64-token chunks: angle addition, segments of two chunks
    (1, 1, 130, 64, 64, 64, 1),     # 64-token chunks, one segment
    (1, 2, 300, 128, 128, 128, 0),  # 128-token chunks: per-row float64 reduction
])
def test_rotation_far_positions(pos0, B, H, N, dk, dv, C, seg):
    """Absolute positions far from zero: the rotation angles must still match the
    oracle's float64 angles (the bf16 kernels reduce the chunk's base angle in
    float64 and add in-chunk offsets in float32)."""
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=N + 7)
    theta = W.rotary_theta(dk)
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(H), theta=to64(theta), pos0=pos0)
    o, st = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=C, theta=theta, pos0=pos0,
                                      return_state=True, segments=seg)
    ref_p = orc.parallel(to64(q), to64(k), to64(v), orc.head_gammas(H), theta=to64(theta), pos0=pos0)
    o_par = R.retention_parallel_fwd(q.to(DEV), k.to(DEV), v.to(DEV), theta=theta, pos0=pos0)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, BF16_TOL, "chunkwise O")
    assert_close(to64(st), ref_s, BF16_TOL, "chunkwise state")
    assert_close(to64(o_par), ref_p, BF16_TOL, "parallel O")


def test_rotation_far_positions_decode_and_f32():
    pos0 = 1_000_000_007
    B, H, dk, dv = 2, 2, 64, 64
    s0, qs, ks, vs = W.make_decode(B, H, dk, dv, torch.float32, 2, 0.01, seed=3)
    theta = W.rotary_theta(dk)
    pos = torch.tensor([pos0, 3 * 2**31 + 5], dtype=torch.int64)
    S = to64(s0)
    state = s0.to(DEV)
    for t in range(2):
        o_ref, S = orc.decode_step(to64(qs[t]), to64(ks[t]), to64(vs[t]), S, orc.head_gammas(H),
                                   theta=to64(theta), pos=(pos + t).numpy())
        o = R.retention_recurrent_step(qs[t].to(DEV), ks[t].to(DEV), vs[t].to(DEV), state, theta=theta,
                                       pos=(pos + t).to(DEV))
        torch.cuda.synchronize()
        assert_close(to64(o), o_ref, F32_TOL, f"decode o step {t}")
    q, k, v = _inputs(1, 2, 150, 64, 64, torch.float32, seed=5)
    ref, _ = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(2), theta=to64(theta), pos0=pos0)
    o = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=64, theta=theta, pos0=pos0)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, F32_TOL, "f32 chunkwise O")


def test_oversize_requests_rejected():
    q, k, v = _inputs(1, 129, 8, 64, 64, torch.bfloat16, seed=1)
    with pytest.raises(RuntimeError):
        R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=64)
    q, k, v = _inputs(1, 1, 8, 64, 1028, torch.bfloat16, seed=1)
    s = torch.zeros((1, 1, 64, 1028), dtype=torch.float32, device=DEV)
    with pytest.raises(RuntimeError):
        R.retention_recurrent_step(q[:, :, 0].contiguous().to(DEV), k[:, :, 0].contiguous().to(DEV),
                                   v[:, :, 0].contiguous().to(DEV), s)


# ------------------------------------------------------------ the full-size workloads


def test_msr_bf16_rotary_full():
    """Multi-scale bf16 workload with rotation, every element."""
    w = W.WORKLOADS["msr_bf16_rotary"]
    q, k, v, theta = W.make_workload("msr_bf16_rotary", device="cpu")
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(w["H"]), theta=to64(theta))
    o, s = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=w["chunk"], theta=theta,
                                     return_state=True)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, BF16_TOL, "O")
    assert_close(to64(s), ref_s, BF16_TOL, "state")


def _sampled_heads_check(q, k, v, o, s, H, heads, theta=None):
    for (b, h) in heads:
        ref, ref_s = orc.recurrent(to64(q[b:b + 1, h:h + 1]), to64(k[b:b + 1, h:h + 1]),
                                   to64(v[b:b + 1, h:h + 1]), orc.head_gammas(H)[h:h + 1],
                                   theta=theta)
        assert_close(to64(o[b:b + 1, h:h + 1]), ref, BF16_TOL, f"O head {(b, h)}")
        if s is not None:
            assert_close(to64(s[b:b + 1, h:h + 1]), ref_s, BF16_TOL, f"state head {(b, h)}")


def test_layer7b_full_sampled_heads():
    w = W.WORKLOADS["layer7b_bf16"]
    q, k, v, _ = W.make_workload("layer7b_bf16", device=DEV)
    o, s = R.retention_chunkwise_fwd(q, k, v, chunk=w["chunk"], return_state=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    _sampled_heads_check(q, k, v, o, s, w["H"], heads=[(0, 0), (3, 15), (2, 7)])


def test_longctx_full_sampled_heads():
    w = W.WORKLOADS["longctx_bf16"]
    q, k, v, _ = W.make_workload("longctx_bf16", device=DEV)
    o, s = R.retention_chunkwise_fwd(q, k, v, chunk=w["chunk"], return_state=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    # every head: this is the workload that runs the two-pass look-back at scale (32 segments in
    # groups), so each chain's flags, slots and decay factors are checked
    _sampled_heads_check(q, k, v, o, s, w["H"], heads=[(0, h) for h in range(w["H"])])


def test_longctx_parallel_crossover_lengths_sampled():
    w = W.WORKLOADS["longctx_bf16"]
    q, k, v, _ = W.make_workload("longctx_bf16", device=DEV)
    for n in w["parallel_lengths"]:
        qn, kn, vn = q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous()
        o_par = R.retention_parallel_fwd(qn, kn, vn)
        o_chk = R.retention_chunkwise_fwd(qn, kn, vn, chunk=w["chunk"])
        torch.cuda.synchronize()
        for h in (1, 6):
            ref = orc.parallel(to64(qn[:, h:h + 1]), to64(kn[:, h:h + 1]), to64(vn[:, h:h + 1]),
                               orc.head_gammas(w["H"])[h:h + 1])
            assert_close(to64(o_par[:, h:h + 1]), ref, BF16_TOL, f"parallel N={n} head {h}")
            assert_close(to64(o_chk[:, h:h + 1]), ref, BF16_TOL, f"chunkwise N={n} head {h}")


def test_decode_full_512_steps_sampled_heads():
    w = W.WORKLOADS["decode_bf16"]
    s0, qs, ks, vs = W.make_decode_workload(device=DEV)
    state = s0.clone()
    heads = [(0, 0), (17, 9), (63, 15)]
    H = w["H"]
    S = {bh: to64(s0[bh[0], bh[1]])[None, None] for bh in heads}
    g = orc.head_gammas(H)
    outs = {bh: [] for bh in heads}
    refs = {bh: [] for bh in heads}
    for t in range(w["steps"]):
        o = R.retention_recurrent_step(qs[t], ks[t], vs[t], state)
        for (b, h) in heads:
            outs[(b, h)].append(o[b, h].float())
    torch.cuda.synchronize()
    qs_c, ks_c, vs_c = qs.cpu(), ks.cpu(), vs.cpu()
    for (b, h) in heads:
        St = S[(b, h)]
        for t in range(w["steps"]):
            o_ref, St = orc.decode_step(to64(qs_c[t, b:b + 1, h:h + 1]), to64(ks_c[t, b:b + 1, h:h + 1]),
                                        to64(vs_c[t, b:b + 1, h:h + 1]), St, g[h:h + 1])
            refs[(b, h)].append(o_ref[0, 0])
        got = torch.stack(outs[(b, h)]).cpu().numpy().astype(np.float64)
        # every step on its own (a wrong step would be diluted in a norm over all 512)
        assert_close(got, np.stack(refs[(b, h)]), BF16_TOL, f"o over 512 steps, head {(b, h)}", per_head_axes=1)
        assert_close(to64(state[b, h]), St[0, 0], BF16_TOL, f"final state head {(b, h)}", per_head_axes=0)


# ------------------------------------------------------------ edge cases and properties


def test_future_inf_key_does_not_leak():
    """The causal mask is a select: an infinite key at the last position must
    not turn earlier outputs into NaN (Inf * 0 would)."""
    B, H, N, dk, dv = 1, 2, 200, 64, 64
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=21)
    k_bad = k.clone()
    k_bad[:, :, -1, :] = float("inf")
    for fn in (lambda a, b, c: R.retention_chunkwise_fwd(a, b, c, chunk=64),
               lambda a, b, c: R.retention_parallel_fwd(a, b, c)):
        good = fn(q.to(DEV), k.to(DEV), v.to(DEV))
        bad = fn(q.to(DEV), k_bad.to(DEV), v.to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(good[:, :, :-1], bad[:, :, :-1])


@pytest.mark.parametrize("shape", [(2, 4, 1000, 128, 128, 128), (1, 2, 4096, 64, 64, 64), (1, 1, 3000, 64, 128, 128)],
                         ids=lambda c: "B{}H{}N{}dk{}dv{}C{}".format(*c))
def test_repeatable_bitwise(shape):
    """Outputs and final states are bitwise identical from call to call, also
    when segments of a head exchange states inside the kernel (the order in
    which segments finish must not change the result)."""
    B, H, N, dk, dv, C = shape
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=5)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    runs = [R.retention_chunkwise_fwd(qd, kd, vd, chunk=C, return_state=True) for _ in range(4)]
    c = R.retention_parallel_fwd(qd, kd, vd)
    d = R.retention_parallel_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    for o, s in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(s, runs[0][1])
    assert torch.equal(c, d)


@pytest.mark.parametrize("N,C,seg", [(500, 128, 3), (2000, 128, 3), (1500, 64, 5)],
                         ids=lambda x: str(x))
def test_state_in_out_alias_segmented(N, C, seg):
    """state_out aliases state_in in a segmented call. With segments longer than
    two chunks (2000 tokens in 3 segments of 768) the two-pass form runs, whose
    first segment reads the initial state a second time while the last one may
    already be done: the final state must not be stored before that read."""
    B, H, dk, dv = 1, 2, 128, 128
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=N + seg)
    s0 = torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(9)) * 0.1
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(H), state0=to64(s0))
    for _ in range(3):
        state = s0.to(DEV).clone()
        o = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=C, state_in=state, state_out=state,
                                      segments=seg)
        torch.cuda.synchronize()
        assert_close(to64(o), ref, BF16_TOL, "O")
        assert_close(to64(state), ref_s, BF16_TOL, "aliased final state")


def test_state_in_out_alias_and_handoff():
    B, H, N, dk, dv = 1, 2, 500, 128, 128
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=33)
    theta = W.rotary_theta(dk)
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(H), theta=to64(theta))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    n1 = 200
    state = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=DEV)
    o1 = R.retention_chunkwise_fwd(qd[:, :, :n1].contiguous(), kd[:, :, :n1].contiguous(),
                                   vd[:, :, :n1].contiguous(), chunk=128, theta=theta, state_in=state,
                                   state_out=state)
    o2 = R.retention_chunkwise_fwd(qd[:, :, n1:].contiguous(), kd[:, :, n1:].contiguous(),
                                   vd[:, :, n1:].contiguous(), chunk=128, theta=theta, pos0=n1, state_in=state,
                                   state_out=state, segments=3)
    torch.cuda.synchronize()
    assert_close(np.concatenate([to64(o1), to64(o2)], axis=2), ref, BF16_TOL, "handed-off O")
    assert_close(to64(state), ref_s, BF16_TOL, "handed-off state")


@pytest.mark.parametrize("gammas", [[1.0, 0.99], [0.5, 0.75], [0.9, 0.999999], [0.3, 0.97], [0.05, 0.6]])
@pytest.mark.parametrize("chunk", [64, 128])
def test_custom_gammas(gammas, chunk):
    """Gammas far from the defaults, including ones small enough (gamma^chunk <
    2^-64) that the chunkwise kernel must use its exact per-element decay
    form instead of the rescaled-values form."""
    B, H, N, dk, dv = 1, 2, 300, 64, 64
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=44)
    g = np.asarray(gammas, dtype=np.float32).astype(np.float64)
    ref = orc.parallel(to64(q), to64(k), to64(v), g)
    for o in (R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=chunk, gamma=list(g)),
              R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=chunk, gamma=list(g), segments=2),
              R.retention_parallel_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gamma=list(g))):
        torch.cuda.synchronize()
        assert_close(to64(o), ref, BF16_TOL, f"gammas {gammas}")


@pytest.mark.parametrize("gammas", [[0.05, 0.6], [0.999, 0.3]])
def test_custom_gammas_f32(gammas):
    """float32 inputs with small gammas: the decay of far-apart query/key blocks
    must not be formed from an overflowing and an underflowing factor."""
    B, H, N, dk, dv = 1, 2, 300, 64, 64
    q, k, v = _inputs(B, H, N, dk, dv, torch.float32, seed=45)
    g = np.asarray(gammas, dtype=np.float32).astype(np.float64)
    ref = orc.parallel(to64(q), to64(k), to64(v), g)
    for o in (R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=64, gamma=list(g)),
              R.retention_parallel_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gamma=list(g))):
        torch.cuda.synchronize()
        assert_close(to64(o), ref, F32_TOL, f"gammas {gammas}")


def test_segment_count_invariance_full_msr():
    w = W.WORKLOADS["msr_bf16_rotary"]
    q, k, v, theta = W.make_workload("msr_bf16_rotary", device=DEV)
    outs = [R.retention_chunkwise_fwd(q, k, v, chunk=w["chunk"], theta=theta, segments=s) for s in (1, 5, 0)]
    torch.cuda.synchronize()
    base = to64(outs[0])
    for o in outs[1:]:
        assert_close(to64(o), base, 5e-3, "segments vs single pass")


def test_workspace_shared_across_sizes():
    """One zero-filled workspace reused by calls of different sizes (different
    chain counts, segment counts and layouts inside the workspace) gives the
    same bits as a fresh workspace per call: nothing an earlier call left in
    it may be taken for a published segment state."""
    cases = [BF16_CHUNK_CASES[i] for i in (0, 1, 3, 4, 5, 0, 4, 1)]
    shared = torch.zeros(48 << 20, dtype=torch.uint8, device=DEV)
    for B, H, N, dk, dv, C, rot, st, seg in cases:
        q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=N + dk + dv)
        q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
        theta = W.rotary_theta(dk) if rot else None
        s0 = (torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(7)) * 0.1).to(DEV) if st else None
        nbytes = R.retention_chunkwise_workspace_size(B, H, N, dk, dv, torch.bfloat16, C, seg)
        assert 0 < nbytes <= shared.numel()
        fresh = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
        kw = dict(chunk=C, theta=theta, pos0=17 if rot else 0, state_in=s0, return_state=True, segments=seg)
        o1, s1 = R.retention_chunkwise_fwd(q, k, v, workspace=fresh, **kw)
        o2, s2 = R.retention_chunkwise_fwd(q, k, v, workspace=shared, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2), (B, H, N, dk, dv, C, seg)


def test_graph_replay_matches_eager():
    """The benchmark replays the step from a HIP graph: every replay, with
    eager work in between, must reproduce the eager result bit for bit."""
    w = W.WORKLOADS["msr_bf16_rotary"]
    q, k, v, theta = W.make_workload("msr_bf16_rotary", device=DEV)
    th = R.HostFloats(theta)
    nbytes = R.retention_chunkwise_workspace_size(w["B"], w["H"], w["N"], w["dk"], w["dv"], q.dtype, w["chunk"])
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    ws2 = torch.zeros_like(ws)
    eager = R.retention_chunkwise_fwd(q, k, v, chunk=w["chunk"], theta=th, workspace=ws)
    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        R.retention_chunkwise_fwd(q, k, v, chunk=w["chunk"], theta=th, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        R.retention_chunkwise_fwd(q, k, v, chunk=w["chunk"], theta=th, out=out, workspace=ws)
    for _ in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        other = R.retention_chunkwise_fwd(q, k, v, chunk=w["chunk"], theta=th, workspace=ws2, segments=3)
        torch.cuda.synchronize()
        assert torch.isfinite(other).all()


# ------------------------------------------------------------ backward

BWD_CASES = [
    # B, H, N, dk, dv, chunk, dtype, rotary, state_in, d_state_out
    (2, 3, 300, 64, 64, 64, torch.bfloat16, False, False, False),
    (1, 2, 333, 128, 128, 128, torch.bfloat16, True, True, True),
    (1, 2, 200, 64, 128, 64, torch.bfloat16, True, False, True),
    (2, 2, 257, 256, 128, 128, torch.bfloat16, False, True, True),
    (1, 2, 1, 64, 64, 64, torch.bfloat16, True, True, True),
    (1, 1, 4100, 64, 64, 64, torch.bfloat16, True, True, True),
    (1, 2, 130, 64, 64, 64, torch.float32, True, True, True),
    (2, 1, 200, 32, 64, 64, torch.float32, False, True, True),
    (1, 2, 700, 64, 64, 256, torch.bfloat16, True, True, True),     # large chunks: one segment per chunk
    (1, 1, 2000, 128, 128, 512, torch.bfloat16, False, True, True),
    (1, 2, 150, 64, 64, 32, torch.float32, True, True, True),       # float32 small chunks
    (1, 2, 300, 64, 512, 64, torch.bfloat16, True, True, True),     # dv = 512: passes 1, 2 over halves of dv
    (2, 2, 257, 256, 512, 128, torch.bfloat16, False, True, True),
    (1, 1, 1100, 128, 256, 128, torch.bfloat16, True, True, True),
]


def _bwd_check(B, H, N, dk, dv, chunk, dtype, rot, st, ds, seed, gamma=None, pos0=None):
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    if pos0 is None:
        pos0 = 11 if rot else 0
    q, k, v = _inputs(B, H, N, dk, dv, dtype, seed)
    d_o, d_s = W.make_upstream_grads(B, H, N, dk, dv, dtype, seed + 1000)
    s0 = W.make_decode(B, H, dk, dv, dtype, 1, 0.1, seed + 2000)[0] if st else None
    theta = W.rotary_theta(dk) if rot else None
    g = _gammas_for(H, gamma)
    ref = orc.backward(to64(q), to64(k), to64(v), to64(d_o), g, theta=None if theta is None else to64(theta),
                       pos0=pos0, state0=None if s0 is None else to64(s0),
                       d_state=to64(d_s) if ds else None)
    got = R.retention_chunkwise_bwd(
        q.to(DEV), k.to(DEV), v.to(DEV), d_o.to(DEV), chunk=chunk, gamma=gamma, theta=theta, pos0=pos0,
        state_in=None if s0 is None else s0.to(DEV), d_state_out=d_s.to(DEV) if ds else None, need_d_state_in=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "d_state_in"), got, ref):
        assert_close(to64(a), b, tol, name)


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}C{}{}rot{}st{}ds{}".format(
    *c[:6], str(c[6])[6:], *c[7:]))
def test_chunkwise_backward_small(case):
    _bwd_check(*case, seed=71)


# 128-token chunks, key widths of 128 or 256 and enough (batch, head, value tile) chains over the
# passes to fill the chip: every pass runs on the wide chunkwise kernel in one launch (the dK and dV
# passes in reverse token order), with ragged last chunks, initial states and state gradients
WIDE_BWD_CASES = [
    # B, H, N, dk, dv, chunk, dtype, rotary, state_in, d_state_out
    (2, 48, 300, 128, 128, 128, torch.bfloat16, True, True, True),    # unsplit; rotation undone afterwards
    (2, 32, 257, 128, 256, 128, torch.bfloat16, False, True, True),   # passes 1, 2 over halves of dv
    (2, 16, 260, 256, 512, 128, torch.bfloat16, True, False, True),   # the 7B-shaped layer's widths
]


@pytest.mark.parametrize("case", WIDE_BWD_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}rot{}".format(*c[:5], c[7]))
def test_chunkwise_backward_wide_passes(case):
    _bwd_check(*case, seed=79)


@pytest.mark.parametrize("pos0", [1_000_000_007, 3 * 2**31 + 5])
@pytest.mark.parametrize("dk,dv,C", [(64, 64, 64), (128, 128, 128), (256, 256, 128)])
def test_chunkwise_backward_rotation_far_positions(pos0, dk, dv, C):
    """dq and dk at absolute positions far from zero. The first two passes rotate
    their output rows back themselves (angle reduced in float64 per row); with
    256-wide keys, 128-column values and 128-token chunks the tile has no LDS
    left for the frequencies and a row kernel rotates them afterwards."""
    _bwd_check(1, 2, 300, dk, dv, C, torch.bfloat16, True, True, True, seed=73, pos0=pos0)


@pytest.mark.parametrize("gammas", [[1.0, 0.99], [0.05, 0.6], [0.9, 0.999999]])
def test_chunkwise_backward_custom_gammas(gammas):
    _bwd_check(1, 2, 700, 64, 64, 64, torch.bfloat16, True, True, True, seed=72, gamma=gammas)


def test_chunkwise_backward_msr_full():
    """The multi-scale bf16 workload with rotation, every element of every gradient."""
    w = W.WORKLOADS["msr_bf16_rotary"]
    _bwd_check(w["B"], w["H"], w["N"], w["dk"], w["dv"], w["chunk"], w["dtype"], True, False, False, seed=w["seed"])


def test_chunkwise_backward_long_d128():
    _bwd_check(1, 2, 4096, 128, 128, 128, torch.bfloat16, False, True, True, seed=73)


def test_chunkwise_backward_leaves_inputs_and_aliases_state():
    B, H, N, dk, dv = 1, 2, 300, 64, 64
    q, k, v = (t.to(DEV) for t in _inputs(B, H, N, dk, dv, torch.bfloat16, 74))
    d_o, d_s = (t.to(DEV) for t in W.make_upstream_grads(B, H, N, dk, dv, torch.bfloat16, 75))
    theta = W.rotary_theta(dk)
    keep = [t.clone() for t in (q, k, v, d_o, d_s)]
    a = R.retention_chunkwise_bwd(q, k, v, d_o, theta=theta, d_state_out=d_s, need_d_state_in=True)
    ds_alias = d_s.clone()
    b = R.retention_chunkwise_bwd(q, k, v, d_o, theta=theta, d_state_out=ds_alias, d_state_in=ds_alias)
    torch.cuda.synchronize()
    for x, y in zip(keep, (q, k, v, d_o, d_s)):
        assert torch.equal(x, y)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    assert torch.equal(a[3], ds_alias)


def test_chunkwise_backward_workspace_needs_no_clearing():
    """One workspace, filled with garbage, serves backward calls of several
    sizes in a row (each clears the counters its passes use)."""
    shapes = [(1, 2, 700, 64, 64, 64), (1, 1, 4100, 64, 64, 64), (2, 2, 300, 128, 128, 128), (1, 2, 700, 64, 64, 64)]
    need = max(R.retention_chunkwise_bwd_workspace_size(B, H, N, dk, dv, torch.bfloat16, C)
               for B, H, N, dk, dv, C in shapes)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    for i, (B, H, N, dk, dv, C) in enumerate(shapes):
        q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, 80 + i)
        d_o, d_s = W.make_upstream_grads(B, H, N, dk, dv, torch.bfloat16, 90 + i)
        g = orc.head_gammas(H)
        ref = orc.backward(to64(q), to64(k), to64(v), to64(d_o), g, d_state=to64(d_s))
        got = R.retention_chunkwise_bwd(q.to(DEV), k.to(DEV), v.to(DEV), d_o.to(DEV), chunk=C,
                                        d_state_out=d_s.to(DEV), need_d_state_in=True, workspace=ws)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "d_state_in"), got, ref):
            assert_close(to64(a), b, BF16_TOL, f"call {i} {name}")


# ------------------------------------------------------------ output stage

EPI_CASES = [
    # B, H, N, dv, d_out, gate, affine
    (2, 3, 50, 64, 128, False, False),
    (2, 3, 50, 64, 128, True, True),
    (1, 2, 300, 128, 256, True, False),
    (1, 1, 130, 256, 128, False, True),
    (1, 2, 77, 512, 384, True, True),
    (3, 4, 129, 64, 640, True, True),
]


def _epi_check(B, H, N, dv, d_out, gate, affine, seed):
    o, w_o, gw, gb, gt = W.make_epilogue(B, H, N, dv, d_out, seed)
    ref = orc.msr_epilogue(to64(o), to64(w_o), gn_weight=to64(gw) if affine else None,
                           gn_bias=to64(gb) if affine else None, gate=to64(gt) if gate else None)
    got = R.retention_msr_epilogue(o.to(DEV), w_o.to(DEV), gn_weight=gw.to(DEV) if affine else None,
                                   gn_bias=gb.to(DEV) if affine else None, gate=gt.to(DEV) if gate else None)
    torch.cuda.synchronize()
    assert_close(to64(got), ref, BF16_TOL, "y", per_head_axes=1)


@pytest.mark.parametrize("case", EPI_CASES, ids=lambda c: "B{}H{}N{}dv{}out{}gate{}aff{}".format(*c))
def test_msr_epilogue_small(case):
    _epi_check(*case, seed=111)


def test_msr_epilogue_msr_full():
    _epi_check(2, 8, 2048, 64, 512, True, True, seed=112)


def test_msr_epilogue_layer7b_sampled_rows():
    """The 7B-shaped layer's output stage (32768 tokens, 16 heads of 512, d_out
    4096) as the benchmark runs it; 96 sampled tokens recomputed by the oracle."""
    B, H, N, dv, d_out = 4, 16, 8192, 512, 4096
    o, w_o, gw, gb, gt = W.make_epilogue(B, H, N, dv, d_out, 113, device=DEV)
    y = R.retention_msr_epilogue(o, w_o, gn_weight=gw, gn_bias=gb, gate=gt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    bs, ns = rng.integers(0, B, 96), rng.integers(0, N, 96)
    ns[:4] = [0, N - 1, 1, N - 2]
    o_s = to64(o[bs, :, ns, :])[:, :, None, :]   # [96, H, 1, dv]: each sampled token as its own batch entry
    ref = orc.msr_epilogue(o_s, to64(w_o), gn_weight=to64(gw), gn_bias=to64(gb), gate=to64(gt[bs, ns])[:, None, :])
    assert_close(to64(y[bs, ns])[:, None, :], ref, BF16_TOL, "sampled rows", per_head_axes=1)


@pytest.mark.parametrize("B,H,dv,d_out", [(64, 16, 512, 4096), (3, 2, 64, 256), (1, 4, 128, 384), (64, 8, 64, 512)])
def test_msr_epilogue_few_rows_split_k(B, H, dv, d_out):
    """At most 64 tokens (a decode step): the projection splits its contraction."""
    _epi_check(B, H, 1, dv, d_out, True, True, seed=114 + B)


STEP_MSR_CASES = [
    # B, H, dk, dv, d_out, rotation. Rows split over step workgroups (B*H < 256 and d_v a
    # multiple of 128) take the separate GroupNorm pass, the others normalise in the step;
    # at most 64 sequences the projection splits K, 65 run the whole-K GEMM.
    (5, 4, 64, 128, 256, False),      # GroupNorm pass, split K
    (5, 4, 64, 128, 256, True),
    (1, 1, 64, 64, 128, False),       # in-step GroupNorm, one head
    (3, 6, 64, 64, 384, True),        # in-step GroupNorm, d_v 64
    (64, 16, 256, 512, 4096, False),  # the decode workload's shape
    (64, 8, 128, 256, 512, True),
    (65, 2, 64, 128, 256, False),     # GroupNorm pass, whole-K GEMM
]


@pytest.mark.parametrize("B,H,dk,dv,d_out,rot", STEP_MSR_CASES)
def test_recurrent_step_msr_matches_oracle(B, H, dk, dv, d_out, rot):
    s0, qs, ks, vs = W.make_decode(B, H, dk, dv, torch.bfloat16, 1, 0.05, seed=120)
    _, w_o, gw, gb, gt = W.make_epilogue(B, H, 1, dv, d_out, 121)
    theta = W.rotary_theta(dk) if rot else None
    pos = torch.tensor([3, 70, 0, 1_000_003, 9] * ((B + 4) // 5), dtype=torch.int64)[:B]
    g = orc.head_gammas(H)
    o_ref, s_ref = orc.decode_step(to64(qs[0]), to64(ks[0]), to64(vs[0]), to64(s0), g,
                                   theta=None if theta is None else to64(theta), pos=pos.numpy() if rot else None)
    y_ref = orc.msr_epilogue(o_ref[:, :, None, :], to64(w_o), gn_weight=to64(gw), gn_bias=to64(gb),
                             gate=to64(gt))[:, 0, :]
    state = s0.to(DEV)
    y, o = R.retention_recurrent_step_msr(qs[0].to(DEV), ks[0].to(DEV), vs[0].to(DEV), state, w_o.to(DEV), theta=theta,
                                          pos=pos.to(DEV) if rot else None, gate=gt[:, 0, :].contiguous().to(DEV),
                                          gn_weight=gw.to(DEV), gn_bias=gb.to(DEV))
    torch.cuda.synchronize()
    assert_close(to64(o), o_ref, BF16_TOL, "o")
    assert_close(to64(state), s_ref, BF16_TOL, "state")
    # the output stage sees the bf16-rounded o the step wrote: compare with the oracle on that o too
    y_on_o = orc.msr_epilogue(to64(o)[:, :, None, :], to64(w_o), gn_weight=to64(gw), gn_bias=to64(gb),
                              gate=to64(gt))[:, 0, :]
    assert_close(to64(y), y_on_o, BF16_TOL, "y (on the step's o)", per_head_axes=0)
    assert_close(to64(y), y_ref, BF16_TOL, "y", per_head_axes=0)


def test_recurrent_step_msr_repeats_bitwise():
    """Consecutive steps reuse the output stage's tickets and partial tiles: the
    same inputs give the same outputs bit for bit, call after call."""
    B, H, dk, dv, d_out = 64, 16, 256, 512, 4096
    s0, qs, ks, vs = W.make_decode(B, H, dk, dv, torch.bfloat16, 1, 0.05, seed=123)
    _, w_o, gw, gb, gt = W.make_epilogue(B, H, 1, dv, d_out, 124)
    args = [x.to(DEV) for x in (qs[0], ks[0], vs[0])]
    kw = dict(gate=gt[:, 0, :].contiguous().to(DEV), gn_weight=gw.to(DEV), gn_bias=gb.to(DEV))
    w_o = w_o.to(DEV)
    outs = []
    for _ in range(4):
        state = s0.to(DEV)
        y, o = R.retention_recurrent_step_msr(*args, state, w_o, **kw)
        outs.append((y.clone(), o.clone(), state))
    torch.cuda.synchronize()
    for y, o, st in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(o, outs[0][1]) and torch.equal(st, outs[0][2])


# ------------------------------------------------------------ large chunks

LARGE_CHUNK_CASES = [
    # B, H, N, dk, dv, chunk, rotary, state_in
    (1, 2, 1000, 64, 64, 256, True, True),
    (2, 2, 700, 128, 128, 512, False, True),
    (1, 1, 3000, 64, 128, 1024, True, False),
    (1, 2, 130, 256, 128, 512, False, True),
    (2, 3, 2100, 64, 64, 384, True, True),
]


@pytest.mark.parametrize("case", LARGE_CHUNK_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}C{}rot{}st{}".format(*c))
def test_chunkwise_large_chunks(case):
    B, H, N, dk, dv, C, rot, st = case
    q, k, v = _inputs(B, H, N, dk, dv, torch.bfloat16, 130)
    theta = W.rotary_theta(dk) if rot else None
    s0 = W.make_decode(B, H, dk, dv, torch.bfloat16, 1, 0.1, 131)[0] if st else None
    g = orc.head_gammas(H)
    ref, ref_s = orc.chunkwise(to64(q), to64(k), to64(v), g, C, theta=None if theta is None else to64(theta), pos0=5,
                               state0=None if s0 is None else to64(s0))
    o, s = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=C, theta=theta, pos0=5,
                                     state_in=None if s0 is None else s0.to(DEV), return_state=True)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, BF16_TOL, "o")
    assert_close(to64(s), ref_s, BF16_TOL, "state")


def test_chunk_size_does_not_change_the_result_msr():
    """The multi-scale workload at chunk 64, 128, 256, 512 and 1024: every result
    within tolerance of the oracle, as all chunk sizes compute the same retention."""
    w = W.WORKLOADS["msr_bf16_rotary"]
    q, k, v, theta = W.make_workload("msr_bf16_rotary", device="cpu")
    ref = orc.parallel(to64(q), to64(k), to64(v), orc.head_gammas(w["H"]), theta=to64(theta))
    for C in (64, 128, 256, 512, 1024):
        o = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=C, theta=theta)
        torch.cuda.synchronize()
        assert_close(to64(o), ref, BF16_TOL, f"chunk {C}")


def test_backward_and_output_stage_graph_replay():
    """The backward (row kernels that also clear its counters, the multi-pass
    launch) and the output stage (GroupNorm, GEMM; and the split-K path) are
    captured in one graph; every replay, with other eager calls in between,
    reproduces the eager results bit for bit."""
    w = W.WORKLOADS["msr_bf16_rotary"]
    q, k, v, theta = W.make_workload("msr_bf16_rotary", device=DEV)
    th = R.HostFloats(theta)
    d_o, d_s = W.make_upstream_grads(w["B"], w["H"], w["N"], w["dk"], w["dv"], w["dtype"], 140, device=DEV)
    o, w_o, gw, gb, gt = W.make_epilogue(w["B"], w["H"], w["N"], w["dv"], 512, 141, device=DEV)
    o1, w1, gw1, gb1, gt1 = W.make_epilogue(16, 8, 1, 64, 512, 142, device=DEV)  # 16 tokens: split-K path
    nb = R.retention_chunkwise_bwd_workspace_size(w["B"], w["H"], w["N"], w["dk"], w["dv"], q.dtype, w["chunk"])
    wsb = torch.full((nb,), 0x5A, dtype=torch.uint8, device=DEV)
    ne = R.retention_msr_epilogue_workspace_size(w["B"], w["H"], w["N"], w["dv"], 512, q.dtype)
    ne1 = R.retention_msr_epilogue_workspace_size(16, 8, 1, 64, 512, q.dtype)
    wse = torch.empty(ne, dtype=torch.uint8, device=DEV)
    wse1 = torch.empty(ne1, dtype=torch.uint8, device=DEV)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dsi = torch.empty((w["B"], w["H"], w["dk"], w["dv"]), dtype=torch.float32, device=DEV)
    y = torch.empty((w["B"], w["N"], 512), dtype=torch.bfloat16, device=DEV)
    y1 = torch.empty((16, 1, 512), dtype=torch.bfloat16, device=DEV)

    def step():
        R.retention_chunkwise_bwd(q, k, v, d_o, chunk=w["chunk"], theta=th, d_state_out=d_s, d_state_in=dsi,
                                  out=grads, workspace=wsb)
        R.retention_msr_epilogue(o, w_o, gn_weight=gw, gn_bias=gb, gate=gt, out=y, workspace=wse)
        R.retention_msr_epilogue(o1, w1, gn_weight=gw1, gn_bias=gb1, gate=gt1, out=y1, workspace=wse1)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (*grads, dsi, y, y1)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        for t in (*grads, dsi, y, y1):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((*grads, dsi, y, y1), eager):
            assert torch.equal(a, b)
        other = R.retention_chunkwise_bwd(q[:, :, :700].contiguous(), k[:, :, :700].contiguous(),
                                          v[:, :, :700].contiguous(), d_o[:, :, :700].contiguous(), theta=th)
        torch.cuda.synchronize()
        assert all(torch.isfinite(t).all() for t in other[:3])


# ------------------------------------------------------------ small chunks

SMALL_CHUNK_CASES = [
    # B, H, N, dk, dv, chunk, dtype, rotary, state_in, segments (float32: its kernel takes any chunk;
    # bf16: 32-token tiles, a 16-token chunk runs on them)
    (1, 2, 150, 64, 64, 16, torch.float32, True, True, 0),
    (2, 1, 130, 32, 64, 32, torch.float32, False, True, 2),
    (1, 3, 300, 64, 128, 32, torch.float32, True, False, 0),
    (1, 2, 333, 64, 64, 32, torch.bfloat16, True, True, 0),
    (2, 3, 200, 128, 192, 32, torch.bfloat16, False, True, 1),
    (1, 2, 1000, 256, 64, 32, torch.bfloat16, True, False, 5),
    (1, 1, 97, 64, 128, 16, torch.bfloat16, False, True, 0),
    (2, 2, 4100, 128, 64, 16, torch.bfloat16, True, True, 0),
]


@pytest.mark.parametrize("case", SMALL_CHUNK_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}C{}{}rot{}st{}seg{}".format(
    *c[:6], str(c[6])[6:], *c[7:]))
def test_chunkwise_small_chunks(case):
    B, H, N, dk, dv, C, dtype, rot, st, seg = case
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    q, k, v = _inputs(B, H, N, dk, dv, dtype, 150)
    theta = W.rotary_theta(dk) if rot else None
    s0 = W.make_decode(B, H, dk, dv, dtype, 1, 0.1, 151)[0] if st else None
    ref, ref_s = orc.chunkwise(to64(q), to64(k), to64(v), orc.head_gammas(H), C,
                               theta=None if theta is None else to64(theta), pos0=9,
                               state0=None if s0 is None else to64(s0))
    o, s = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=C, theta=theta, pos0=9,
                                     state_in=None if s0 is None else s0.to(DEV), return_state=True, segments=seg)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, tol, "o")
    assert_close(to64(s), ref_s, tol, "state")




def test_chunkwise_backward_layer7b_sampled_heads():
    """The 7B-shaped layer's backward (B=4 H=16 N=8192 d_k=256 d_v=512, chunk 128: the
    passes keyed by d_v run over its halves) as the benchmark runs it; two sampled
    (batch, head) pairs recomputed by the oracle."""
    w = W.WORKLOADS["layer7b_bf16"]
    q, k, v, _ = W.make_workload("layer7b_bf16", device=DEV)
    d_o, _ = W.make_upstream_grads(w["B"], w["H"], w["N"], w["dk"], w["dv"], w["dtype"], w["seed"] + 1000, device=DEV)
    dq, dk_, dv_, _ = R.retention_chunkwise_bwd(q, k, v, d_o, chunk=w["chunk"])
    torch.cuda.synchronize()
    g = orc.head_gammas(w["H"])
    for b, h in ((0, 0), (3, 13)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = orc.backward(to64(q[sl]), to64(k[sl]), to64(v[sl]), to64(d_o[sl]), [g[h]])
        for name, got, r in zip(("dq", "dk", "dv"), (dq[sl], dk_[sl], dv_[sl]), ref):
            assert_close(to64(got), r, BF16_TOL, f"{name} (b={b}, h={h})")
