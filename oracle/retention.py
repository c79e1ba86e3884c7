"""Plain fp64 CPU oracle for multi-scale retention (RetNet's retention).

TEST INFRASTRUCTURE. Only the test suite, the smoke check in the graft entry
point and the CPU-baseline leg of the benchmark import this module. The
product path (the HIP library and its Python binding) never imports, calls or
links it, and this module imports nothing from the product: it shares no code,
table or constant with the GPU kernels. Inputs are plain numpy arrays; every
computation is numpy in float64, written to be checked against the pages by eye.

What is computed, per batch b and head h, on the exact input values upcast to
float64 (pages: "RetNet Guide: Retentive Networks & The Impossible Triangle",
sections "The Parallel Representation for High-Throughput Pretraining",
"The Recurrent Representation for Constant-Memory O(1) Decoding" and "The
Chunkwise Recurrent Representation for Ultra-Long Sequence Prefill"; and "How
RetNet Combines Parallel Training and Constant Inference"):

    o_n = sum_{m <= n} gamma_h^(n - m) (q'_n . k'_m) v_m

where q', k' are the query/key rows after the optional complex rotation. The
three forms the pages give (parallel, recurrent, chunkwise) are implemented
separately below so that their agreement is itself a check.

Readings taken where the pages are silent, ambiguous or defective:
  * heads are counted from 0, so head h decays with 1 - 2^(-5-h) and a single
    head uses 1 - 2^-5 (the guide's PyTorch listing counts from 0; its formula
    text says h in {1..H});
  * no 1/sqrt(d) score scale (the formulas carry none; callers fold any scale
    into q);
  * the chunk carry printed in the guide's chunkwise section omits the decay
    of each key inside the chunk. The carry used here weights key j of a chunk
    of length L by gamma^(L-1-j), which is what the recurrent form implies;
  * the cross-chunk row factor gamma^(j+1) uses 0-based j inside the chunk;
  * rotation: consecutive coordinates (2j, 2j+1) form the complex number
    x_2j + i x_2j+1, which is multiplied by e^(i n theta_j) at absolute
    position n, for queries and keys alike; the score is the real dot product
    of the rotated real vectors, i.e. Re(z_q conj(z_k) e^(i (n-m) theta)).
    Pairing adjacent coordinates (rather than first half with second half) is
    a convention the pages do not fix;
  * positions are absolute and 0-based: token t of a call sits at pos0 + t.

Parity status: every public function here is pinned by tests that do not
restate it (hand-worked values, the decay widget's printed gamma and
half-life, cross-form agreement, textbook special cases, invariants; the
backward by hand-worked values, finite differences, which are exact here
because the loss is affine in each single input entry, and homogeneity; the
output stage by a hand-worked value, torch's GroupNorm and linear layer, and
the per-group mean and variance). The
adjacent-pair rotation convention is a documented choice, not something a
printed value decides.
"""

import numpy as np

__all__ = [
    "head_gammas",
    "half_life",
    "rotate_pairs",
    "decay_matrix",
    "parallel",
    "recurrent",
    "chunkwise",
    "segmented",
    "decode_step",
    "backward",
    "msr_epilogue",
]


def head_gammas(num_heads):
    """Per-head decay gamma_h = 1 - 2^(-5-h), h = 0..H-1.

    "RetNet Guide" section "3. Multi-Scale Retention (MSR): Hierarchical
    Temporal Decay" gives the formula; "RetNet" (siftaillc) "Multi-scale
    decay: drag a head" gives the same rule. Heads counted from 0.
    """
    h = np.arange(num_heads, dtype=np.float64)
    return 1.0 - np.exp2(-5.0 - h)


def half_life(gamma):
    """Tokens until a weight gamma^n falls to one half: ln(1/2) / ln(gamma).

    The siftaillc "Multi-scale decay" widget prints a head's gamma together
    with this half-life.
    """
    return np.log(0.5) / np.log(np.asarray(gamma, dtype=np.float64))


def rotate_pairs(x, positions, theta):
    """Complex rotation of the last axis of x by e^(i * position * theta_j).

    x: [..., N, d] with d even; positions: [N] absolute positions; theta: [d/2].
    Coordinates (2j, 2j+1) are the real and imaginary parts of one complex
    number ("RetNet Guide" section "2. Relative Position via Complex
    Exponential Phase Rotations"; "How RetNet Combines ..." likens it to RoPE).
    """
    x = np.asarray(x, dtype=np.float64)
    theta = np.asarray(theta, dtype=np.float64)
    d = x.shape[-1]
    if d % 2 != 0 or theta.shape != (d // 2,):
        raise ValueError("rotation needs an even last axis and d/2 frequencies")
    angle = np.outer(np.asarray(positions, dtype=np.float64), theta)  # [N, d/2]
    c = np.cos(angle)
    s = np.sin(angle)
    re = x[..., 0::2]
    im = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = re * c - im * s
    out[..., 1::2] = re * s + im * c
    return out


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def _maybe_rotate(q, k, theta, pos0):
    if theta is None:
        return q, k
    n = q.shape[-2]
    positions = pos0 + np.arange(n, dtype=np.float64)
    return rotate_pairs(q, positions, theta), rotate_pairs(k, positions, theta)


def decay_matrix(gamma, n):
    """D[i, j] = gamma^(i-j) for i >= j, else 0 (an n x n matrix).

    "RetNet Guide" section "1. The Parallel Representation for High-Throughput
    Pretraining", definition of the causal decay matrix D.
    """
    idx = np.arange(n)
    dist = idx[:, None] - idx[None, :]
    return np.where(dist >= 0, np.power(float(gamma), np.maximum(dist, 0)), 0.0)


def parallel(q, k, v, gammas, theta=None, pos0=0):
    """Parallel form O = ((Q K^T) * D) V, one head at a time.

    q, k: [B, H, N, dk]; v: [B, H, N, dv]; gammas: [H]. Returns O [B, H, N, dv].
    "RetNet Guide", parallel representation; "RetNet" (siftaillc)
    "One mechanism, three shapes": Retention(X) = (Q K^T (.) D) V.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    q, k = _maybe_rotate(q, k, theta, pos0)
    B, H, N, _ = q.shape
    out = np.empty(v.shape, dtype=np.float64)
    for h in range(H):
        D = decay_matrix(gammas[h], N)
        for b in range(B):
            scores = q[b, h] @ k[b, h].T
            out[b, h] = (scores * D) @ v[b, h]
    return out


def recurrent(q, k, v, gammas, theta=None, pos0=0, state0=None):
    """Recurrent form, one token at a time.

    S_n = gamma S_{n-1} + k_n^T v_n ; o_n = q_n S_n  ("RetNet Guide" section
    "2. The Recurrent Representation for Constant-Memory O(1) Decoding";
    "How RetNet Combines ...": decay the previous state, add the current
    key-value product, query the updated state).
    Returns (O [B, H, N, dv], S_N [B, H, dk, dv]). state0 defaults to zeros.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    q, k = _maybe_rotate(q, k, theta, pos0)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if state0 is None else _as64(state0).copy()
    g = np.asarray(gammas, dtype=np.float64)[None, :, None, None]
    out = np.empty((B, H, N, dv), dtype=np.float64)
    for n in range(N):
        S = g * S + k[:, :, n, :, None] * v[:, :, n, None, :]
        out[:, :, n, :] = np.einsum("bhi,bhij->bhj", q[:, :, n, :], S)
    return out, S


def chunkwise(q, k, v, gammas, chunk, theta=None, pos0=0, state0=None):
    """Chunkwise recurrent form: parallel inside a chunk, state carried across.

    For a chunk X of length L (the last may be short) with carried state S:
      O_X = ((Q_X K_X^T) * D_L) V_X + zeta * (Q_X S),   zeta_j = gamma^(j+1)
      S  <- gamma^L S + K_X^T (xi * V_X),               xi_j   = gamma^(L-1-j)
    ("RetNet Guide" section "3. The Chunkwise Recurrent Representation";
    the xi weights are the correction of its printed carry, see module doc.)
    Returns (O, S_final).
    """
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    q, k, v = _as64(q), _as64(k), _as64(v)
    q, k = _maybe_rotate(q, k, theta, pos0)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if state0 is None else _as64(state0).copy()
    out = np.empty((B, H, N, dv), dtype=np.float64)
    for start in range(0, N, chunk):
        L = min(chunk, N - start)
        sl = slice(start, start + L)
        j = np.arange(L, dtype=np.float64)
        for h in range(H):
            g = float(gammas[h])
            D = decay_matrix(g, L)
            zeta = np.power(g, j + 1.0)[:, None]
            xi = np.power(g, L - 1.0 - j)[:, None]
            for b in range(B):
                Qc, Kc, Vc = q[b, h, sl], k[b, h, sl], v[b, h, sl]
                inner = ((Qc @ Kc.T) * D) @ Vc
                cross = zeta * (Qc @ S[b, h])
                out[b, h, sl] = inner + cross
                S[b, h] = (g ** L) * S[b, h] + Kc.T @ (xi * Vc)
    return out, S


def segmented(q, k, v, gammas, chunk, segment_len, theta=None, pos0=0, state0=None):
    """Chunkwise form run per segment after a scan of segment end states.

    The sequence is cut into segments of segment_len tokens (a multiple of
    chunk; the last may be short). (1) each segment's end state T_s is built
    from a zero state with the chunk carry; (2) the start state of segment s
    is the scan S_in(s) = gamma^segment_len S_in(s-1) + T_{s-1}, S_in(0) =
    state0; (3) every segment runs the chunkwise form from S_in(s). This is
    the chunk-to-chunk carry law of "RetNet Guide" section "3. The Chunkwise
    Recurrent Representation" applied to runs of chunks.
    Returns (O, S_final).
    """
    if segment_len < 1 or segment_len % chunk != 0:
        raise ValueError("segment_len must be a positive multiple of chunk")
    q, k, v = _as64(q), _as64(k), _as64(v)
    q, k = _maybe_rotate(q, k, theta, pos0)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    starts = list(range(0, N, segment_len))
    zero = np.zeros((B, H, dk, dv))
    ends = []
    for s0 in starts:
        sl = slice(s0, min(N, s0 + segment_len))
        _, T = chunkwise(q[:, :, sl], k[:, :, sl], v[:, :, sl], gammas, chunk, state0=zero)
        ends.append(T)
    g_seg = np.power(np.asarray(gammas, dtype=np.float64), segment_len)[None, :, None, None]
    S_in = [zero.copy() if state0 is None else _as64(state0).copy()]
    for s in range(1, len(starts)):
        S_in.append(g_seg * S_in[s - 1] + ends[s - 1])
    out = np.empty((B, H, N, dv), dtype=np.float64)
    S_final = None
    for s, s0 in enumerate(starts):
        sl = slice(s0, min(N, s0 + segment_len))
        out[:, :, sl], S_final = chunkwise(
            q[:, :, sl], k[:, :, sl], v[:, :, sl], gammas, chunk, state0=S_in[s]
        )
    if S_final is None:
        S_final = zero if state0 is None else _as64(state0).copy()
    return out, S_final


def decode_step(q, k, v, state, gammas, theta=None, pos=None):
    """One recurrent decode step for one token per sequence.

    q, k: [B, H, dk]; v: [B, H, dv]; state: [B, H, dk, dv]; pos: [B] absolute
    positions (needed only with theta). Returns (o [B, H, dv], new state).
    S <- gamma S + k^T v ; o = q S ("RetNet Guide", recurrent representation;
    its listing's forward_recurrent returns the output and the new state).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    if theta is not None:
        if pos is None:
            raise ValueError("rotation needs positions")
        pos = np.asarray(pos, dtype=np.float64)
        q = np.stack([rotate_pairs(q[b][:, None, :], [pos[b]], theta)[:, 0, :]
                      for b in range(q.shape[0])])
        k = np.stack([rotate_pairs(k[b][:, None, :], [pos[b]], theta)[:, 0, :]
                      for b in range(k.shape[0])])
    g = np.asarray(gammas, dtype=np.float64)[None, :, None, None]
    S = g * _as64(state) + k[:, :, :, None] * v[:, :, None, :]
    o = np.einsum("bhi,bhij->bhj", q, S)
    return o, S


def backward(q, k, v, d_o, gammas, theta=None, pos0=0, state0=None, d_state=None):
    """Gradients of one retention call with respect to all of its inputs.

    The call is the one `recurrent` computes: O [B, H, N, dv] and the final
    state S_N [B, H, dk, dv] from q, k [B, H, N, dk], v [B, H, N, dv] and the
    initial state state0 (None = zeros). Given the gradients d_o of O and
    d_state of S_N (None = zeros), returns (dq, dk, dv, d_state0).

    Training evaluates the whole sequence at once in the parallel form ("RetNet
    Guide" section "1. The Parallel Representation for High-Throughput
    Pretraining"; "Retentive Networks (RetNet)" (krlt), "At a glance": training
    parallel over the sequence), so its backward is that of the parallel form.
    Per head, with Q', K' the rotated rows, D the decay matrix,
    Z_n = gamma^(n+1) and Xi_m = gamma^(N-1-m) (0-based n, m):
        O   = ((Q' K'^T) * D) V + Z * (Q' S0)
        S_N = gamma^N S0 + K'^T (Xi * V)
    and differentiating each term:
        dV  = ((Q' K'^T) * D)^T dO + Xi * (K' dS)
        dQ' = ((dO V^T) * D) K' + Z * (dO S0^T)
        dK' = ((dO V^T) * D)^T Q' + Xi * (V dS^T)
        dS0 = Q'^T (Z * dO) + gamma^N dS
    The rotation multiplies each pair by a unit complex number, so its adjoint
    is the rotation by the opposite angle: dQ = rotate(dQ', -theta), and the
    same for dK.
    """
    q, k, v, d_o = _as64(q), _as64(k), _as64(v), _as64(d_o)
    qr, kr = _maybe_rotate(q, k, theta, pos0)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if state0 is None else _as64(state0)
    dS = np.zeros((B, H, dk, dv)) if d_state is None else _as64(d_state)
    n = np.arange(N, dtype=np.float64)
    dq_r = np.empty_like(qr)
    dk_r = np.empty_like(kr)
    dv_out = np.empty_like(v)
    dS0 = np.empty_like(S0)
    for h in range(H):
        g = float(gammas[h])
        D = decay_matrix(g, N)
        Z = np.power(g, n + 1.0)[:, None]
        Xi = np.power(g, N - 1.0 - n)[:, None]
        for b in range(B):
            Qh, Kh, Vh, dOh = qr[b, h], kr[b, h], v[b, h], d_o[b, h]
            P = (Qh @ Kh.T) * D
            dP = (dOh @ Vh.T) * D
            dv_out[b, h] = P.T @ dOh + Xi * (Kh @ dS[b, h])
            dq_r[b, h] = dP @ Kh + Z * (dOh @ S0[b, h].T)
            dk_r[b, h] = dP.T @ Qh + Xi * (Vh @ dS[b, h].T)
            dS0[b, h] = Qh.T @ (Z * dOh) + (g ** N) * dS[b, h]
    if theta is not None:
        positions = pos0 + n
        minus = -np.asarray(theta, dtype=np.float64)
        dq_r = rotate_pairs(dq_r, positions, minus)
        dk_r = rotate_pairs(dk_r, positions, minus)
    return dq_r, dk_r, dv_out, dS0


def msr_epilogue(o, w_o, gn_weight=None, gn_bias=None, gate=None, eps=1e-6):
    """Multi-scale retention's output stage: GroupNorm of the concatenated heads,
    an optional gate, and the output projection.

    "RetNet Guide" section "1. The Parallel Representation for High-Throughput
    Pretraining" writes MSR(X) = GroupNorm(Concat(R_1, ..., R_H)) W_O; its
    listing normalises with one group per head (eps 1e-6, per-channel weight
    and bias) and projects with a bias-free linear layer whose weight is
    [d_out, H*dv]. "How RetNet Combines ..." names a gating step applied with
    the GroupNorm but gives no formula: here the gate is an optional tensor the
    caller supplies, multiplied element by element after the GroupNorm.

    o: [B, H, N, dv] retention outputs; w_o: [d_out, H*dv]; gn_weight, gn_bias:
    [H*dv] (None: ones / zeros); gate: [B, N, H*dv] or None.
    Returns y [B, N, d_out] = (GroupNorm(concat) * gate) w_o^T.
    """
    o = _as64(o)
    B, H, N, dv = o.shape
    x = np.transpose(o, (0, 2, 1, 3))  # [B, N, H, dv]: the heads of one token side by side
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)  # biased, over the head's dv channels
    z = ((x - mean) / np.sqrt(var + eps)).reshape(B, N, H * dv)
    if gn_weight is not None:
        z = z * _as64(gn_weight)
    if gn_bias is not None:
        z = z + _as64(gn_bias)
    if gate is not None:
        z = z * _as64(gate)
    return z @ _as64(w_o).T
