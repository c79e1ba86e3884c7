"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each check would fail on a plausible mistake in the oracle: hand-worked values
(decay direction, causal inclusion of m = n, rotation sign), the decay widget's
printed gamma and half-life, agreement of independently written forms
(parallel / recurrent / chunkwise / segmented), textbook special cases
(cumulative linear attention at gamma = 1, orthonormal-key recall) and
invariants (linearity, relative position, state hand-off, fixed state size).
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import retention as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- decay table


def test_decay_widget_gamma_and_half_life():
    w = _load("decay_widget.json")
    g = orc.head_gammas(8)
    # the widget's head: printed to 6 decimals, with a ~177-token half-life
    matches = [h for h in range(8) if round(float(g[h]), 6) == w["printed_gamma_6dp"]]
    assert matches == [3]
    assert round(float(orc.half_life(g[3]))) == w["printed_half_life_tokens"]
    # single-head workload quotes 1 - 2^-5 for its only head (heads count from 0)
    assert orc.head_gammas(1)[0] == w["single_head_gamma"]


def test_gammas_increase_towards_one_and_are_fp32_exact():
    g = orc.head_gammas(16)
    assert np.all(np.diff(g) > 0) and np.all(g < 1.0) and np.all(g > 0.96)
    assert np.array_equal(g.astype(np.float32).astype(np.float64), g)
    # half-life doubles (to first order) from one head to the next
    hl = orc.half_life(g)
    assert np.allclose(hl[1:] / hl[:-1], 2.0, rtol=0.02)


# ------------------------------------------------------------ hand-worked values


def _single(x):
    return np.asarray(x, dtype=np.float64).reshape(1, 1, len(x), -1)


@pytest.mark.parametrize("form", ["parallel", "recurrent", "chunk1", "chunk2", "segmented"])
def test_hand_worked_decay(form):
    ex = _load("hand_worked.json")["decay"]
    q, k, v = _single(ex["q"]), _single(ex["k"]), _single(ex["v"])
    g = np.array([ex["gamma"]])
    if form == "parallel":
        o = orc.parallel(q, k, v, g)
        S = None
    elif form == "recurrent":
        o, S = orc.recurrent(q, k, v, g)
    elif form == "chunk1":
        o, S = orc.chunkwise(q, k, v, g, 1)
    elif form == "chunk2":
        o, S = orc.chunkwise(q, k, v, g, 2)
    else:
        o, S = orc.segmented(q, k, v, g, 1, 2)
    assert np.allclose(o.ravel(), ex["o"], rtol=0, atol=1e-15)
    if S is not None:
        assert abs(float(S.ravel()[0]) - ex["state"]) < 1e-15


def test_hand_worked_rotation():
    ex = _load("hand_worked.json")["rotation"]
    q = np.array(ex["q"])[None, None]
    k = np.array(ex["k"])[None, None]
    v = np.array(ex["v"])[None, None]
    th = np.array(ex["theta"])
    rq = orc.rotate_pairs(q, [0, 1], th)[0, 0]
    rk = orc.rotate_pairs(k, [0, 1], th)[0, 0]
    assert np.allclose(rq, ex["rotated_q_pos0_0"], atol=1e-15)
    assert np.allclose(rk, ex["rotated_k_pos0_0"], atol=1e-15)
    for gam, key in ((1.0, "o_gamma_1"), (0.5, "o_gamma_half")):
        for pos0 in (0, 1, 7):
            o_par = orc.parallel(q, k, v, np.array([gam]), theta=th, pos0=pos0)
            o_rec, _ = orc.recurrent(q, k, v, np.array([gam]), theta=th, pos0=pos0)
            assert np.allclose(o_par[0, 0], ex[key], atol=1e-12)
            assert np.allclose(o_rec[0, 0], ex[key], atol=1e-12)


def test_hand_worked_decode():
    ex = _load("hand_worked.json")["decode"]
    S = np.full((1, 1, 1, 1), ex["state0"])
    g = np.array([ex["gamma"]])
    for (qq, kk, vv), o_exp, s_exp in zip(ex["steps"], ex["o"], ex["state"]):
        o, S = orc.decode_step(np.full((1, 1, 1), qq), np.full((1, 1, 1), kk),
                               np.full((1, 1, 1), vv), S, g)
        assert float(o.ravel()[0]) == o_exp
        assert float(S.ravel()[0]) == s_exp


# ------------------------------------------------------------ cross-form agreement


@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 16, 37, 64])
@pytest.mark.parametrize("rot", [False, True])
def test_three_forms_agree(chunk, rot):
    B, H, N, dk, dv = 2, 3, 37, 8, 6
    q, k, v = _rand((B, H, N, dk), 1), _rand((B, H, N, dk), 2), _rand((B, H, N, dv), 3)
    g = np.array([0.9, 0.97, 0.999])
    th = 10000.0 ** (-2.0 * np.arange(dk // 2) / dk) if rot else None
    o_par = orc.parallel(q, k, v, g, theta=th, pos0=5)
    o_rec, s_rec = orc.recurrent(q, k, v, g, theta=th, pos0=5)
    o_chk, s_chk = orc.chunkwise(q, k, v, g, chunk, theta=th, pos0=5)
    scale = np.abs(o_par).max()
    assert np.abs(o_rec - o_par).max() < 1e-12 * scale
    assert np.abs(o_chk - o_par).max() < 1e-12 * scale
    assert np.abs(s_chk - s_rec).max() < 1e-12 * np.abs(s_rec).max()


@pytest.mark.parametrize("chunk,seg", [(2, 4), (4, 8), (5, 10), (3, 36)])
def test_segmented_scan_matches_recurrent(chunk, seg):
    B, H, N, dk, dv = 1, 2, 37, 6, 4
    q, k, v = _rand((B, H, N, dk), 4), _rand((B, H, N, dk), 5), _rand((B, H, N, dv), 6)
    s0 = _rand((B, H, dk, dv), 7)
    g = np.array([0.8, 0.99])
    o_rec, s_rec = orc.recurrent(q, k, v, g, state0=s0)
    o_seg, s_seg = orc.segmented(q, k, v, g, chunk, seg, state0=s0)
    assert np.abs(o_seg - o_rec).max() < 1e-12 * np.abs(o_rec).max()
    assert np.abs(s_seg - s_rec).max() < 1e-12 * np.abs(s_rec).max()


def test_printed_chunk_carry_needs_key_decay():
    """The guide's chunkwise carry as printed (no in-chunk key decay) differs
    from the recurrent form when gamma < 1 and agrees only at gamma = 1; the
    oracle's corrected carry agrees in both cases."""

    def printed_carry(q, k, v, g, C):
        N = q.shape[0]
        S = np.zeros((q.shape[1], v.shape[1]))
        out = np.empty((N, v.shape[1]))
        for s in range(0, N, C):
            Q, K, V = q[s:s + C], k[s:s + C], v[s:s + C]
            L = Q.shape[0]
            j = np.arange(L)
            D = np.where(j[:, None] >= j[None, :], g ** np.maximum(j[:, None] - j[None, :], 0), 0)
            out[s:s + C] = ((Q @ K.T) * D) @ V + (g ** (j + 1))[:, None] * (Q @ S)
            S = g ** L * S + K.T @ V
        return out

    N, dk, dv = 12, 4, 3
    q, k, v = _rand((N, dk), 8), _rand((N, dk), 9), _rand((N, dv), 10)
    for g, should_match in ((0.9, False), (1.0, True)):
        ref, _ = orc.recurrent(q[None, None], k[None, None], v[None, None], np.array([g]))
        lit = printed_carry(q, k, v, g, 4)
        fixed, _ = orc.chunkwise(q[None, None], k[None, None], v[None, None], np.array([g]), 4)
        assert np.allclose(fixed[0, 0], ref[0, 0], atol=1e-12)
        assert np.allclose(lit, ref[0, 0], atol=1e-9) == should_match


# ------------------------------------------------------------ special cases


def test_gamma_one_is_cumulative_linear_attention():
    """gamma = 1 and identity feature map: the linear-attention recurrence
    s_t = s_{t-1} + k_t^T v_t, o_t = q_t s_t of the guide's 'Low-Cost
    Inference' paragraph, here evaluated with numpy's cumulative sum."""
    B, H, N, dk, dv = 2, 2, 19, 5, 7
    q, k, v = _rand((B, H, N, dk), 11), _rand((B, H, N, dk), 12), _rand((B, H, N, dv), 13)
    outer = k[..., :, None] * v[..., None, :]  # [B,H,N,dk,dv]
    states = np.cumsum(outer, axis=2)
    expect = np.einsum("bhni,bhnij->bhnj", q, states)
    g = np.ones(H)
    for o in (orc.parallel(q, k, v, g), orc.recurrent(q, k, v, g)[0], orc.chunkwise(q, k, v, g, 4)[0]):
        assert np.allclose(o, expect, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gamma", [1.0, 0.9])
def test_orthonormal_key_recall(gamma):
    """Querying with a stored key returns its value exactly for orthonormal keys
    at gamma = 1 ('perfect recall' claim, restricted), and gamma^(n-m) times it
    otherwise."""
    d, dv, N = 8, 5, 8
    Qm, _ = np.linalg.qr(_rand((d, d), 14))
    keys = Qm.T[:N]  # orthonormal rows
    vals = _rand((N, dv), 15)
    for m in range(N - 1):
        q = np.zeros((N, d))
        q[N - 1] = keys[m]
        o, _ = orc.recurrent(q[None, None], keys[None, None], vals[None, None], np.array([gamma]))
        assert np.allclose(o[0, 0, N - 1], gamma ** (N - 1 - m) * vals[m], atol=1e-12)


def test_single_token_and_heads_independent():
    B, H, dk, dv = 2, 3, 4, 5
    q, k, v = _rand((B, H, 1, dk), 16), _rand((B, H, 1, dk), 17), _rand((B, H, 1, dv), 18)
    g = orc.head_gammas(H)
    o = orc.parallel(q, k, v, g)
    assert np.allclose(o[..., 0, :], np.sum(q * k, -1) * v[..., 0, :], atol=1e-14)
    q, k, v = _rand((B, H, 9, dk), 19), _rand((B, H, 9, dk), 20), _rand((B, H, 9, dv), 21)
    full, _ = orc.recurrent(q, k, v, g)
    for h in range(H):
        one, _ = orc.recurrent(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], g[h:h + 1])
        assert np.allclose(one[:, 0], full[:, h], atol=1e-14)


def test_zero_theta_is_no_rotation():
    q, k, v = _rand((1, 2, 11, 6), 22), _rand((1, 2, 11, 6), 23), _rand((1, 2, 11, 3), 24)
    g = orc.head_gammas(2)
    a = orc.parallel(q, k, v, g, theta=np.zeros(3), pos0=123)
    b = orc.parallel(q, k, v, g)
    assert np.allclose(a, b, atol=1e-14)


# ------------------------------------------------------------ invariants


def test_linearity():
    q, k, v = _rand((1, 2, 13, 4), 25), _rand((1, 2, 13, 4), 26), _rand((1, 2, 13, 3), 27)
    v2 = _rand((1, 2, 13, 3), 28)
    g = orc.head_gammas(2)
    o1, o2 = orc.parallel(q, k, v, g), orc.parallel(q, k, v2, g)
    assert np.allclose(orc.parallel(q, k, 2 * v - 3 * v2, g), 2 * o1 - 3 * o2, atol=1e-12)
    assert np.allclose(orc.parallel(-1.5 * q, k, v, g), -1.5 * o1, atol=1e-12)


def test_rotation_norm_and_relative_position():
    x = _rand((3, 17, 10), 29)
    th = _rand((5,), 30)
    pos = np.arange(17) * 37.0 + 5
    r = orc.rotate_pairs(x, pos, th)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # score between positions n and m depends only on n - m
    a, b = _rand((10,), 31), _rand((10,), 32)
    s1 = orc.rotate_pairs(a[None], [50.0], th)[0] @ orc.rotate_pairs(b[None], [20.0], th)[0]
    s2 = orc.rotate_pairs(a[None], [1030.0], th)[0] @ orc.rotate_pairs(b[None], [1000.0], th)[0]
    assert abs(s1 - s2) < 1e-10


def test_state_handoff_and_fixed_state_size():
    B, H, N, dk, dv = 1, 2, 40, 6, 5
    q, k, v = _rand((B, H, N, dk), 33), _rand((B, H, N, dk), 34), _rand((B, H, N, dv), 35)
    g = orc.head_gammas(H)
    th = 10000.0 ** (-2.0 * np.arange(dk // 2) / dk)
    o_all, s_all = orc.chunkwise(q, k, v, g, 8, theta=th)
    n1 = 13
    o_a, s_a = orc.chunkwise(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], g, 8, theta=th)
    o_b, s_b = orc.chunkwise(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], g, 8, theta=th,
                             pos0=n1, state0=s_a)
    assert np.allclose(np.concatenate([o_a, o_b], axis=2), o_all, atol=1e-12)
    assert np.allclose(s_b, s_all, atol=1e-12)
    # the carried state has the same size whatever the length
    for n in (1, 7, 40):
        _, s = orc.recurrent(q[:, :, :n], k[:, :, :n], v[:, :, :n], g)
        assert s.shape == (B, H, dk, dv)


def test_decode_closed_form():
    """After n steps, S_n = gamma^n S_0 + sum_m gamma^(n-m) k_m^T v_m, and each
    step's output equals the recurrent form started from S_0."""
    B, H, dk, dv, n = 2, 3, 5, 4, 9
    g = orc.head_gammas(H)
    S0 = _rand((B, H, dk, dv), 36)
    qs, ks, vs = _rand((n, B, H, dk), 37), _rand((n, B, H, dk), 38), _rand((n, B, H, dv), 39)
    S = S0
    outs = []
    for t in range(n):
        o, S = orc.decode_step(qs[t], ks[t], vs[t], S, g)
        outs.append(o)
    gg = g[None, :, None, None]
    expect = gg ** n * S0 + sum(gg ** (n - 1 - m) * ks[m][..., :, None] * vs[m][..., None, :]
                                for m in range(n))
    assert np.allclose(S, expect, atol=1e-12)
    o_rec, _ = orc.recurrent(np.moveaxis(qs, 0, 2), np.moveaxis(ks, 0, 2),
                             np.moveaxis(vs, 0, 2), g, state0=S0)
    assert np.allclose(np.stack(outs, axis=2), o_rec, atol=1e-12)


def test_decode_rotation_matches_sequence_form():
    B, H, dk, dv = 2, 2, 6, 3
    g = orc.head_gammas(H)
    th = 10000.0 ** (-2.0 * np.arange(dk // 2) / dk)
    q, k, v = _rand((B, H, 1, dk), 40), _rand((B, H, 1, dk), 41), _rand((B, H, 1, dv), 42)
    S0 = _rand((B, H, dk, dv), 43)
    pos = np.array([3, 250])
    o, S = orc.decode_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], S0, g, theta=th, pos=pos)
    for b in range(B):
        o_r, s_r = orc.recurrent(q[b:b + 1], k[b:b + 1], v[b:b + 1], g, theta=th,
                                 pos0=int(pos[b]), state0=S0[b:b + 1])
        assert np.allclose(o[b], o_r[0, :, 0], atol=1e-13)
        assert np.allclose(S[b], s_r[0], atol=1e-13)


def test_brute_force_scalar_loops():
    """Scalar pure-Python evaluation of the definition on tiny shapes."""
    rng = np.random.default_rng(44)
    for trial in range(6):
        N, dk, dv = int(rng.integers(1, 7)), 2 * int(rng.integers(1, 3)), int(rng.integers(1, 4))
        gam = float(rng.uniform(0.5, 1.0))
        th = rng.uniform(0, 3, dk // 2)
        pos0 = int(rng.integers(0, 50))
        q, k, v = rng.standard_normal((N, dk)), rng.standard_normal((N, dk)), rng.standard_normal((N, dv))

        def rot(x, n):
            y = list(x)
            for j in range(dk // 2):
                a, b = x[2 * j], x[2 * j + 1]
                c, s = math.cos(n * th[j]), math.sin(n * th[j])
                y[2 * j], y[2 * j + 1] = a * c - b * s, a * s + b * c
            return y

        expect = np.zeros((N, dv))
        for n in range(N):
            qn = rot(q[n], pos0 + n)
            for m in range(n + 1):
                km = rot(k[m], pos0 + m)
                score = sum(qn[i] * km[i] for i in range(dk)) * gam ** (n - m)
                for c in range(dv):
                    expect[n, c] += score * v[m, c]
        got = orc.chunkwise(q[None, None], k[None, None], v[None, None], np.array([gam]), 2,
                            theta=th, pos0=pos0)[0][0, 0]
        assert np.allclose(got, expect, atol=1e-12)


# ---------------------------------------------------------------- backward


def test_backward_hand_worked():
    # One head, d_k = d_v = 1, two tokens, gamma = 1/2, worked by hand from
    #   o_0 = g q0 s + q0 k0 v0,  o_1 = g^2 q1 s + q1 (g k0 v0 + k1 v1),
    #   S_2 = g^2 s + g k0 v0 + k1 v1,
    # with q = (1, 2), k = (3, -1), v = (1/2, 2), s = 4, dO = (1, -2), dS = 3:
    #   dq = (dO0 (k0 v0 + g s), dO1 (g k0 v0 + k1 v1 + g^2 s))     = (3.5, 0.5)
    #   dk = (dO0 q0 v0 + dO1 g q1 v0 + g dS v0, dO1 q1 v1 + dS v1) = (0.25, -2)
    #   dv = (dO0 q0 k0 + dO1 g q1 k0 + g k0 dS, dO1 q1 k1 + k1 dS) = (1.5, 1)
    #   ds = g q0 dO0 + g^2 q1 dO1 + g^2 dS                         = 0.25
    q, k, v = _single([1.0, 2.0]), _single([3.0, -1.0]), _single([0.5, 2.0])
    d_o = _single([1.0, -2.0])
    s0 = np.full((1, 1, 1, 1), 4.0)
    ds = np.full((1, 1, 1, 1), 3.0)
    dq, dk, dv, dS0 = orc.backward(q, k, v, d_o, [0.5], state0=s0, d_state=ds)
    assert np.allclose(dq.ravel(), [3.5, 0.5], atol=1e-15)
    assert np.allclose(dk.ravel(), [0.25, -2.0], atol=1e-15)
    assert np.allclose(dv.ravel(), [1.5, 1.0], atol=1e-15)
    assert np.allclose(dS0.ravel(), [0.25], atol=1e-15)
    # without the state terms only the products inside the sequence remain
    dq, dk, dv, dS0 = orc.backward(q, k, v, d_o, [0.5])
    assert np.allclose(dq.ravel(), [1.5, 2.5], atol=1e-15)
    assert np.allclose(dk.ravel(), [-0.5, -8.0], atol=1e-15)
    assert np.allclose(dv.ravel(), [-3.0, 4.0], atol=1e-15)
    assert np.allclose(dS0.ravel(), [-0.5], atol=1e-15)


def _loss(q, k, v, s0, d_o, ds, g, th, pos0):
    o, sn = orc.recurrent(q, k, v, g, theta=th, pos0=pos0, state0=s0)
    return float(np.sum(d_o * o) + np.sum(ds * sn))


@pytest.mark.parametrize("rot", [False, True])
def test_backward_matches_finite_differences(rot):
    # <dO, O> + <dS, S_N> is affine in every single input entry, so a central
    # difference is exact up to rounding for any step: no truncation error.
    B, H, N, dk, dv = 1, 2, 5, 4, 3
    q, k = _rand((B, H, N, dk), 41), _rand((B, H, N, dk), 42)
    v = _rand((B, H, N, dv), 43)
    s0 = _rand((B, H, dk, dv), 44)
    d_o, ds = _rand((B, H, N, dv), 45), _rand((B, H, dk, dv), 46)
    g = [0.8, 0.55]
    th = _rand((dk // 2,), 47) if rot else None
    pos0 = 7 if rot else 0
    got = orc.backward(q, k, v, d_o, g, theta=th, pos0=pos0, state0=s0, d_state=ds)
    args = [q, k, v, s0]
    for which, grad in enumerate(got):
        x = args[which]
        fd = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            hi = [a.copy() for a in args]
            lo = [a.copy() for a in args]
            hi[which][idx] += 0.5
            lo[which][idx] -= 0.5
            fd[idx] = _loss(*hi, d_o, ds, g, th, pos0) - _loss(*lo, d_o, ds, g, th, pos0)
        assert np.allclose(grad, fd, rtol=1e-9, atol=1e-10), which


def test_backward_euler_identities():
    # The loss <dO, O> + <dS, S_N> is homogeneous of degree one in q, in k, in
    # v and in the initial state taken one at a time (except that the state
    # also reaches S_N): sum(x * dx) splits the loss into its terms.
    B, H, N, dk, dv = 2, 2, 23, 6, 5
    q, k = _rand((B, H, N, dk), 51), _rand((B, H, N, dk), 52)
    v, s0 = _rand((B, H, N, dv), 53), _rand((B, H, dk, dv), 54)
    d_o, ds = _rand((B, H, N, dv), 55), _rand((B, H, dk, dv), 56)
    g, th = orc.head_gammas(H), _rand((dk // 2,), 57)
    o, sn = orc.recurrent(q, k, v, g, theta=th, pos0=3, state0=s0)
    o_seq, sn_seq = orc.recurrent(q, k, v, g, theta=th, pos0=3)  # terms without the initial state
    dq, dk_, dv_, dS0 = orc.backward(q, k, v, d_o, g, theta=th, pos0=3, state0=s0, d_state=ds)
    loss = np.sum(d_o * o) + np.sum(ds * sn)
    seq_part = np.sum(d_o * o_seq) + np.sum(ds * sn_seq)
    assert np.isclose(np.sum(q * dq), np.sum(d_o * o), rtol=1e-11)
    assert np.isclose(np.sum(k * dk_), seq_part, rtol=1e-11)
    assert np.isclose(np.sum(v * dv_), seq_part, rtol=1e-11)
    assert np.isclose(np.sum(s0 * dS0), loss - seq_part, rtol=1e-11)


def test_backward_gamma_one_is_cumulative_sums():
    # gamma = 1, no rotation, no state: dV_m = K_m (sum_{n >= m} Q_n^T dO_n) and
    # dQ_n = dO_n (sum_{m <= n} V_m^T K_m), suffix and prefix sums of outer
    # products (the gradient of cumulative linear attention).
    q, k = _rand((1, 1, 9, 3), 61), _rand((1, 1, 9, 3), 62)
    v, d_o = _rand((1, 1, 9, 2), 63), _rand((1, 1, 9, 2), 64)
    dq, dk, dv, _ = orc.backward(q, k, v, d_o, [1.0])
    Q, K, V, G = q[0, 0], k[0, 0], v[0, 0], d_o[0, 0]
    for n in range(9):
        pre = sum(np.outer(V[m], K[m]) for m in range(n + 1))
        suf_qg = sum(np.outer(Q[t], G[t]) for t in range(n, 9))
        assert np.allclose(dq[0, 0, n], G[n] @ pre, atol=1e-12)
        assert np.allclose(dv[0, 0, n], K[n] @ suf_qg, atol=1e-12)
        assert np.allclose(dk[0, 0, n], suf_qg @ V[n], atol=1e-12)


# ---------------------------------------------------------------- MSR epilogue


def test_epilogue_hand_worked():
    # one head, dv = 2, one token (1, 3): mean 2, biased variance 1, so with
    # eps = 0 the normalised row is (-1, 1); weight (2, 3), bias (1, 0) give
    # (-1, 3); gate (1, 0.5) gives (-1, 1.5); w_o = [[1, 1], [2, -1]] gives
    # (0.5, -3.5).
    o = np.array([1.0, 3.0]).reshape(1, 1, 1, 2)
    y = orc.msr_epilogue(o, [[1.0, 1.0], [2.0, -1.0]], gn_weight=[2.0, 3.0], gn_bias=[1.0, 0.0],
                         gate=np.array([1.0, 0.5]).reshape(1, 1, 2), eps=0.0)
    assert np.allclose(y.ravel(), [0.5, -3.5], atol=1e-15)


def test_epilogue_matches_torch_group_norm_and_linear():
    # torch's GroupNorm over [tokens, channels] with one group per head is the
    # listing's normalisation; the oracle computes it by hand
    torch = pytest.importorskip("torch")
    B, H, N, dv, d_out = 2, 3, 7, 8, 5
    o = _rand((B, H, N, dv), 101)
    w_o, wt, bs = _rand((d_out, H * dv), 102), _rand((H * dv,), 103), _rand((H * dv,), 104)
    gate = _rand((B, N, H * dv), 105)
    got = orc.msr_epilogue(o, w_o, gn_weight=wt, gn_bias=bs, gate=gate)
    x = torch.from_numpy(np.transpose(o, (0, 2, 1, 3)).reshape(B * N, H * dv))
    gn = torch.nn.functional.group_norm(x, H, torch.from_numpy(wt), torch.from_numpy(bs), eps=1e-6)
    ref = torch.nn.functional.linear(gn * torch.from_numpy(gate.reshape(B * N, H * dv)), torch.from_numpy(w_o))
    assert np.allclose(got.reshape(B * N, d_out), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_epilogue_normalises_each_head_of_each_token():
    # identity projection, no affine, no gate: every (token, head) group has
    # mean 0 and variance var / (var + eps); with eps = 0 the result does not
    # change when a head's outputs are scaled or shifted
    B, H, N, dv = 1, 4, 6, 16
    o = _rand((B, H, N, dv), 106) * np.arange(1, H + 1)[None, :, None, None]
    eye = np.eye(H * dv)
    y = orc.msr_epilogue(o, eye, eps=1e-6).reshape(B, N, H, dv)
    x = np.transpose(o, (0, 2, 1, 3))
    var = x.var(axis=-1)
    assert np.allclose(y.mean(axis=-1), 0.0, atol=1e-12)
    assert np.allclose(y.var(axis=-1), var / (var + 1e-6), rtol=1e-12)
    o2 = o * 3.5 + 2.0
    assert np.allclose(orc.msr_epilogue(o2, eye, eps=0.0), orc.msr_epilogue(o, eye, eps=0.0), atol=1e-12)
