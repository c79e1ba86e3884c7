"""GPU parity of the wide-head chunkwise kernel (d_k 128 or 256, value tiles of
128 columns, 128-token chunks, one pass per head) against the fp64 oracle.

The library takes this kernel for bf16 calls without rotation; `segments=1`
forces one pass per head for small shapes, and more segments run its
three-kernel form (segment end states from zero, their scan, the segments from
their start states).
The cases cross its decay groups (up to 8 chunks of 128 tokens between two
rescalings of the carried state), end in ragged chunks, carry states in and
out, and use gammas that select each group length (and one that the kernel
does not take, which the general kernel then serves).
"""

import numpy as np
import pytest
import torch

import linear_attention_sequence_fwd_amd as R
from linear_attention_sequence_fwd_amd import workloads as W
from oracle import retention as orc

from helpers import BF16_TOL, assert_close, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    R.load_library()
    yield
    torch.cuda.synchronize()


def _run(B, H, N, dk, dv, st, gammas, seed, segments=1):
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, seed, device="cpu")
    s0 = torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(seed + 1)) * 0.1 if st else None
    g = orc.head_gammas(H) if gammas is None else np.asarray(gammas, dtype=np.float64)
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), g, state0=None if s0 is None else to64(s0))
    o, s = R.retention_chunkwise_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunk=128,
                                     gamma=None if gammas is None else list(gammas),
                                     state_in=None if s0 is None else s0.to(DEV), return_state=True,
                                     segments=segments)
    torch.cuda.synchronize()
    return o, s, ref, ref_s


WIDE_CASES = [
    # B, H, N, dk, dv, state_in
    (1, 2, 300, 128, 128, True),
    (2, 1, 1, 256, 128, True),
    (1, 2, 128, 256, 256, False),
    (2, 2, 129, 256, 128, True),
    (1, 1, 1100, 256, 512, True),
    (1, 3, 2600, 128, 256, False),
    (1, 2, 2048, 256, 128, False),
    (3, 2, 777, 128, 384, True),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}st{}".format(*c))
def test_wide_chunkwise_matches_oracle(case):
    B, H, N, dk, dv, st = case
    o, s, ref, ref_s = _run(B, H, N, dk, dv, st, None, seed=N + dk + dv)
    assert_close(to64(o), ref, BF16_TOL, "O")
    assert_close(to64(s), ref_s, BF16_TOL, "state")


# group lengths: 1.0 with 0.9 -> 2 chunks; 0.999999 with 0.75 -> 1 chunk;
# 0.6 -> gamma^128 < 2^-64, served by the general kernel
@pytest.mark.parametrize("gammas", [[1.0, 0.9], [0.999999, 0.75], [0.6, 0.99], [0.97, 0.96875]])
def test_wide_custom_gammas(gammas):
    o, s, ref, ref_s = _run(1, 2, 1500, 256, 128, True, gammas, seed=11)
    assert_close(to64(o), ref, BF16_TOL, "O")
    assert_close(to64(s), ref_s, BF16_TOL, "state")


def test_wide_repeatable_bitwise():
    q, k, v = W.make_qkv(2, 2, 1000, 256, 256, torch.bfloat16, 5, device=DEV)
    runs = [R.retention_chunkwise_fwd(q, k, v, chunk=128, return_state=True, segments=1) for _ in range(3)]
    torch.cuda.synchronize()
    for o, s in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(s, runs[0][1])


def test_wide_state_alias_and_handoff():
    """Two calls hand the state over in one buffer (state_out aliases state_in)."""
    B, H, N, dk, dv = 1, 2, 1300, 256, 128
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, 21, device="cpu")
    ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(H))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    n1 = 700
    state = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=DEV)
    o1 = R.retention_chunkwise_fwd(qd[:, :, :n1].contiguous(), kd[:, :, :n1].contiguous(),
                                   vd[:, :, :n1].contiguous(), chunk=128, state_in=state, state_out=state,
                                   segments=1)
    o2 = R.retention_chunkwise_fwd(qd[:, :, n1:].contiguous(), kd[:, :, n1:].contiguous(),
                                   vd[:, :, n1:].contiguous(), chunk=128, pos0=n1, state_in=state,
                                   state_out=state, segments=1)
    torch.cuda.synchronize()
    assert_close(np.concatenate([to64(o1), to64(o2)], axis=2), ref, BF16_TOL, "handed-off O")
    assert_close(to64(state), ref_s, BF16_TOL, "handed-off state")


def test_wide_output_leaves_neighbours_untouched():
    """A ragged last chunk stores only its valid rows: a guard tail placed
    right after the output keeps its contents."""
    B, H, N, dk, dv = 1, 2, 200, 256, 128
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, 3, device=DEV)
    o = torch.full((B * H * N + 64, dv), 7.0, dtype=torch.bfloat16, device=DEV)
    view = o[: B * H * N].view(B, H, N, dv)
    R.retention_chunkwise_fwd(q, k, v, chunk=128, segments=1, out=view)
    torch.cuda.synchronize()
    assert torch.all(o[B * H * N:] == 7.0)
    ref, _ = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(H))
    assert_close(to64(view), ref, BF16_TOL, "O")


SEG_CASES = [
    # B, H, N, dk, dv, segments, state_in
    (1, 2, 300, 128, 128, 2, True),     # a short last segment
    (1, 2, 129, 128, 128, 2, True),     # a last segment of one token
    (1, 1, 1100, 256, 512, 3, True),
    (1, 3, 2600, 128, 256, 5, False),
    (2, 1, 777, 256, 128, 4, True),
    (1, 1, 4096, 128, 128, 32, False),  # one chunk per segment
    (1, 2, 5000, 256, 128, 3, True),    # segments of 13 chunks: two decay groups and a ragged one
]


def _segmented_plan(B, H, N, dk, dv, segments):
    import ctypes

    class Plan(ctypes.Structure):
        _fields_ = [(n, ctypes.c_int) for n in ("tile", "dv_tile", "value_tiles", "segments", "segment_len",
                                                 "group_len", "segments_max", "reserved")] + \
                   [(n, ctypes.c_uint64) for n in ("flags_off", "gflags_off", "agg_off", "gagg_off",
                                                    "workspace_bytes")]
    p = Plan()
    assert R.load_library().retention_chunkwise_plan(B, H, N, dk, dv, 1, 128, segments, ctypes.byref(p)) == 0
    return p


@pytest.mark.parametrize("case", SEG_CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}seg{}st{}".format(*c))
def test_wide_segmented_matches_oracle(case):
    B, H, N, dk, dv, seg, st = case
    p = _segmented_plan(B, H, N, dk, dv, seg)
    assert p.segments > 1 and p.tile == 128 and p.dv_tile == 128  # the three-kernel form runs
    o, s, ref, ref_s = _run(B, H, N, dk, dv, st, None, seed=N + seg, segments=seg)
    assert_close(to64(o), ref, BF16_TOL, "O")
    assert_close(to64(s), ref_s, BF16_TOL, "state")


@pytest.mark.parametrize("gammas", [[1.0, 0.9], [0.999999, 0.75], [0.97, 0.96875]])
def test_wide_segmented_custom_gammas(gammas):
    o, s, ref, ref_s = _run(1, 2, 3000, 128, 128, True, gammas, seed=13, segments=4)
    assert_close(to64(o), ref, BF16_TOL, "O")
    assert_close(to64(s), ref_s, BF16_TOL, "state")


def test_wide_segmented_repeatable_and_alias():
    """Bit-for-bit repeats (the scan and every segment run in a fixed order), and
    state_out aliasing state_in: the last segment writes the final state after
    the scan has read the initial one."""
    B, H, N, dk, dv = 1, 2, 2500, 256, 256
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, 8, device=DEV)
    s0 = torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(9)) * 0.1
    runs = [R.retention_chunkwise_fwd(q, k, v, chunk=128, state_in=s0.to(DEV), return_state=True, segments=5)
            for _ in range(3)]
    state = s0.to(DEV).clone()
    o_alias = R.retention_chunkwise_fwd(q, k, v, chunk=128, state_in=state, state_out=state, segments=5)
    torch.cuda.synchronize()
    for o, s in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(s, runs[0][1])
    assert torch.equal(o_alias, runs[0][0]) and torch.equal(state, runs[0][1])
    ref, ref_s = orc.recurrent(to64(q.cpu()), to64(k.cpu()), to64(v.cpu()), orc.head_gammas(H), state0=to64(s0))
    assert_close(to64(runs[0][0]), ref, BF16_TOL, "O")
    assert_close(to64(runs[0][1]), ref_s, BF16_TOL, "state")
