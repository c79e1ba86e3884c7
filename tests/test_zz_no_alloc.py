"""The allocation-free chunkwise entry point against the ordinary one.

retention_chunkwise_fwd_noalloc keeps the segmented form's workspace in a
device array of the library instead of a caller's buffer. Called through the
C ABI twice in a row (the second call smaller, so it reuses what the first
left in the array), it must give bit for bit the ordinary entry point's
results, which the other GPU tests hold to the oracle.
"""

import pytest
import torch

import linear_attention_sequence_fwd_amd as R
from linear_attention_sequence_fwd_amd import workloads as W
from oracle import retention as orc

from helpers import BF16_TOL, assert_close, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pair(B, H, N, dk, dv, C, rot, st, seg, seed):
    q, k, v = W.make_qkv(B, H, N, dk, dv, torch.bfloat16, seed, device=DEV)
    theta = W.rotary_theta(dk) if rot else None
    s0 = torch.randn((B, H, dk, dv), generator=torch.Generator().manual_seed(seed), dtype=torch.float32)
    s0 = (s0 * 0.1).to(DEV) if st else None
    o_ref, s_ref = R.retention_chunkwise_fwd(q, k, v, chunk=C, theta=theta, pos0=5, state_in=s0, return_state=True,
                                             segments=seg)
    out = torch.full_like(v, float("nan"))
    s_out = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device=DEV)
    R.retention_chunkwise_fwd_noalloc(q, k, v, out, chunk=C, theta=theta, pos0=5, state_in=s0, state_out=s_out,
                                      segments=seg)
    torch.cuda.synchronize()
    return q, k, v, theta, s0, o_ref, s_ref, out, s_out


def test_noalloc_matches_workspace_call_twice():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    R.load_library()
    cases = [
        # the multi-scale workload (segmented, local pass: 16 segments per head)
        (2, 8, 2048, 64, 64, 64, True, False, 0, 2),
        # smaller: another shape through the same array (two-pass segments, state in)
        (1, 2, 900, 128, 128, 128, False, True, 3, 3),
    ]
    for i, case in enumerate(cases):
        q, k, v, theta, s0, o_ref, s_ref, out, s_out = _pair(*case)
        assert torch.equal(out, o_ref), f"call {i}: outputs differ"
        assert torch.equal(s_out, s_ref), f"call {i}: final states differ"
        if i == 1:  # and the oracle agrees
            B, H = case[0], case[1]
            ref, ref_s = orc.recurrent(to64(q), to64(k), to64(v), orc.head_gammas(H), pos0=5, state0=to64(s0))
            assert_close(to64(out), ref, BF16_TOL, "O")
            assert_close(to64(s_out), ref_s, BF16_TOL, "state")


def test_noalloc_rejects_plans_beyond_its_array():
    # 4096 chunks of 512 tokens, each a segment with its own published state: far beyond the array
    B, H, N, dk, dv = 1, 1, 4096 * 512, 128, 128
    ws = R.retention_chunkwise_workspace_size(B, H, N, dk, dv, torch.bfloat16, 512)
    assert ws > (32 << 20)
    q = torch.empty((B, H, 16, dk), dtype=torch.bfloat16, device=DEV)  # never read: the call is rejected first
    lib = R.load_library()
    st = lib.retention_chunkwise_fwd_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), B, H, N, dk, dv,
                                             1, 512, None, None, 0, None, None, 0, None)
    assert st == 6  # RET_ERR_WORKSPACE
