"""GPU parity of the single-wave-per-SIMD parallel-form kernel (heads without
rotation, d_k 64 or 128, d_v a multiple of 128) against the fp64 oracle.

The library takes this kernel for bf16 retention_parallel_fwd calls without
theta at those widths. The cases end in ragged query and key blocks (N around
multiples of 128, and N = 1), cross several value tiles, and use gammas small
enough that the walk over key blocks stops early (every decay factor of the
earlier blocks underflows float32) next to gammas of 1 and nearly 1.
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


CASES = [
    # B, H, N, dk, dv
    (1, 2, 1, 128, 128),
    (2, 1, 127, 64, 128),
    (1, 2, 128, 128, 256),
    (1, 3, 129, 128, 128),
    (2, 2, 300, 64, 256),
    (1, 2, 1000, 128, 128),
    (1, 1, 2100, 128, 384),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}dk{}dv{}".format(*c))
def test_parallel_wide_matches_oracle(case):
    B, H, N, dk, dv = case
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, 7 * N + dk + dv, device="cpu")
    ref = orc.parallel(to64(q), to64(k), to64(v), orc.head_gammas(H))
    o = R.retention_parallel_fwd(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert_close(to64(o), ref, BF16_TOL, "O")


# 0.5 and 0.05: the walk stops after one or two key blocks; 1.0: no decay at all
@pytest.mark.parametrize("gammas", [[0.5, 0.05], [1.0, 0.999999], [0.9, 0.96875]])
def test_parallel_wide_custom_gammas(gammas):
    B, H, N, dk, dv = 1, 2, 700, 128, 128
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, 19, device="cpu")
    ref = orc.parallel(to64(q), to64(k), to64(v), np.asarray(gammas, dtype=np.float64))
    o = R.retention_parallel_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gamma=gammas)
    torch.cuda.synchronize()
    assert_close(to64(o), ref, BF16_TOL, "O")


def test_parallel_wide_agrees_with_chunkwise_and_leaves_neighbours_untouched():
    """The parallel and chunkwise forms of one call agree, and a ragged last
    query block stores only its rows (a guard tail after the output keeps its
    contents)."""
    B, H, N, dk, dv = 1, 2, 333, 128, 256
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, 23, device=DEV)
    o = torch.full((B * H * N + 64, dv), 3.0, dtype=torch.bfloat16, device=DEV)
    view = o[: B * H * N].view(B, H, N, dv)
    R.retention_parallel_fwd(q, k, v, out=view)
    oc = R.retention_chunkwise_fwd(q, k, v, chunk=128)
    torch.cuda.synchronize()
    assert torch.all(o[B * H * N:] == 3.0)
    ref = orc.parallel(to64(q), to64(k), to64(v), orc.head_gammas(H))
    assert_close(to64(view), ref, BF16_TOL, "parallel O")
    assert_close(to64(oc), ref, BF16_TOL, "chunkwise O")


# (B, H, N, dk, dv): 4096 tokens of 8 heads (the long-context heads: 32 query blocks a head, walks
# longer than 16 split); 2100 tokens over three value tiles (17 blocks, T = 9); 1000 tokens (8 blocks,
# T = 4) with d_k 64 and two value tiles
BALANCED = [(1, 8, 4096, 128, 128), (1, 1, 2100, 128, 384), (2, 1, 1000, 64, 256)]


@pytest.mark.parametrize("case", BALANCED, ids=lambda c: "B{}H{}N{}dk{}dv{}".format(*c))
def test_parallel_wide_balanced_schedule(case):
    """The split schedule (two workgroups per long walk, partials added by the later one) agrees with
    the oracle and with whole walks, repeats bit for bit over calls that reuse the workspace, and
    leaves the workspace ready (its counters back at zero)."""
    B, H, N, dk, dv = case
    assert R.retention_parallel_workspace_size(B, H, N, dk, dv, torch.bfloat16) > 0
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, 31 + N, device=DEV)
    whole = R.retention_parallel_fwd(q, k, v, balanced=False)
    runs = [R.retention_parallel_fwd(q, k, v) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert torch.equal(r, runs[0])
    assert_close(to64(runs[0]), to64(whole), BF16_TOL, "balanced vs whole walks")
    # the oracle on sampled heads (the whole tensor at the smaller sizes)
    heads = range(H) if N * H <= 4096 else [0, H // 2, H - 1]
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    g = orc.head_gammas(H)
    for h in heads:
        ref = orc.parallel(to64(qc[:, h:h + 1]), to64(kc[:, h:h + 1]), to64(vc[:, h:h + 1]), g[h:h + 1])
        assert_close(to64(runs[0][:, h:h + 1].cpu()), ref, BF16_TOL, "O head %d" % h)


def test_parallel_wide_balanced_guard_tail():
    """A split schedule with a ragged last query block stores only its rows."""
    B, H, N, dk, dv = 1, 2, 1333, 128, 128
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, 41, device=DEV)
    o = torch.full((B * H * N + 64, dv), 3.0, dtype=torch.bfloat16, device=DEV)
    view = o[: B * H * N].view(B, H, N, dv)
    R.retention_parallel_fwd(q, k, v, out=view)
    torch.cuda.synchronize()
    assert torch.all(o[B * H * N:] == 3.0)
    ref = orc.parallel(to64(q), to64(k), to64(v), orc.head_gammas(H))
    assert_close(to64(view), ref, BF16_TOL, "O")


def test_parallel_wide_workspace_shared_across_sizes():
    """A split call after a larger one on the same workspace (the larger call's partials lie where a
    layout sized by the call would put the smaller call's tickets) is still right."""
    for B, H, N, dk, dv in [(1, 8, 4096, 128, 128), (1, 2, 700, 128, 128), (1, 1, 300, 64, 128)]:
        q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, 57 + N, device=DEV)
        o = R.retention_parallel_fwd(q, k, v)
        torch.cuda.synchronize()
        h = H - 1
        ref = orc.parallel(to64(q[:, h:h + 1]), to64(k[:, h:h + 1]), to64(v[:, h:h + 1]), orc.head_gammas(H)[h:h + 1])
        assert_close(to64(o[:, h:h + 1]), ref, BF16_TOL, "O at N=%d" % N)
