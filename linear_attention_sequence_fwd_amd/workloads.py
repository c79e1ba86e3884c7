"""Seeded synthetic workloads for retention (inputs only).

This module holds the workload table and the seeded draws of Q, K, V, the
rotary frequencies and the decode state. It contains none of retention's own
arithmetic (no decay, no rotation, no contraction), so the HIP path and the
fp64 oracle can both be fed from it without sharing any of the method.

Draw recipe: a torch.Generator on the target device seeded with the workload's
seed draws float32 N(0, 1) tensors in the fixed order Q, K, V (then, for
decode, S_0 and the per-step q, k, v), each scaled by 1/sqrt(d_k) and rounded
to the workload's dtype. Rotary frequencies are theta_j = 10000^(-2j/d_k).
"""

import math

import torch

# The five workloads: single-head fp32 correctness case, multi-scale bf16 with
# rotation, a 7B-shaped layer, batched decode, and a long-context prefill.
WORKLOADS = {
    "single_head_f32": dict(B=1, H=1, N=256, dk=64, dv=64, dtype=torch.float32, chunk=64, rotary=False,
                            seed=1),
    "msr_bf16_rotary": dict(B=2, H=8, N=2048, dk=64, dv=64, dtype=torch.bfloat16, chunk=64, rotary=True,
                            seed=2),
    "layer7b_bf16": dict(B=4, H=16, N=8192, dk=256, dv=512, dtype=torch.bfloat16, chunk=128, rotary=False,
                         seed=3),
    "decode_bf16": dict(B=64, H=16, dk=256, dv=512, dtype=torch.bfloat16, steps=512, state_std=0.01,
                        rotary=False, seed=4),
    "longctx_bf16": dict(B=1, H=8, N=65536, dk=128, dv=128, dtype=torch.bfloat16, chunk=128, rotary=False,
                         seed=5, parallel_lengths=(512, 1024, 2048, 4096)),
}


def rotary_theta(dk):
    """theta_j = 10000^(-2j/dk), j = 0 .. dk/2 - 1, as float32 values."""
    return torch.tensor([10000.0 ** (-2.0 * j / dk) for j in range(dk // 2)], dtype=torch.float32)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_qkv(B, H, N, dk, dv, dtype, seed, device="cpu"):
    """Q, K [B,H,N,dk] and V [B,H,N,dv]: N(0,1)/sqrt(dk) drawn in float32, then cast."""
    g = _gen(device, seed)
    scale = 1.0 / math.sqrt(dk)
    q = torch.randn((B, H, N, dk), generator=g, device=device, dtype=torch.float32).mul_(scale).to(dtype)
    k = torch.randn((B, H, N, dk), generator=g, device=device, dtype=torch.float32).mul_(scale).to(dtype)
    v = torch.randn((B, H, N, dv), generator=g, device=device, dtype=torch.float32).mul_(scale).to(dtype)
    return q, k, v


def make_workload(name, device="cpu", N=None):
    """Inputs of a named workload (optionally truncated/extended to length N)."""
    w = WORKLOADS[name]
    n = w["N"] if N is None else N
    q, k, v = make_qkv(w["B"], w["H"], n, w["dk"], w["dv"], w["dtype"], w["seed"], device)
    theta = rotary_theta(w["dk"]) if w.get("rotary") else None
    return q, k, v, theta


def make_decode(B, H, dk, dv, dtype, steps, state_std, seed, device="cpu"):
    """Decode inputs: S_0 ~ N(0, state_std^2) float32 [B,H,dk,dv] and per-step
    q, k [steps,B,H,dk], v [steps,B,H,dv] ~ N(0,1)/sqrt(dk) in dtype."""
    g = _gen(device, seed)
    s0 = torch.randn((B, H, dk, dv), generator=g, device=device, dtype=torch.float32).mul_(state_std)
    scale = 1.0 / math.sqrt(dk)
    q = torch.randn((steps, B, H, dk), generator=g, device=device, dtype=torch.float32).mul_(scale).to(dtype)
    k = torch.randn((steps, B, H, dk), generator=g, device=device, dtype=torch.float32).mul_(scale).to(dtype)
    v = torch.randn((steps, B, H, dv), generator=g, device=device, dtype=torch.float32).mul_(scale).to(dtype)
    return s0, q, k, v


def make_decode_workload(name="decode_bf16", device="cpu", steps=None):
    w = WORKLOADS[name]
    return make_decode(w["B"], w["H"], w["dk"], w["dv"], w["dtype"], steps or w["steps"], w["state_std"],
                       w["seed"], device)


def make_upstream_grads(B, H, N, dk, dv, dtype, seed, device="cpu"):
    """Gradients arriving at a retention call from the layers after it, for
    the backward: dO [B,H,N,dv] ~ N(0,1) in dtype and dS [B,H,dk,dv] ~ N(0,1)
    float32 (the gradient of the final state, as when the next piece of a
    sequence continued from it)."""
    g = _gen(device, seed)
    d_o = torch.randn((B, H, N, dv), generator=g, device=device, dtype=torch.float32).to(dtype)
    d_s = torch.randn((B, H, dk, dv), generator=g, device=device, dtype=torch.float32)
    return d_o, d_s


def make_epilogue(B, H, N, dv, d_out, seed, device="cpu", dtype=torch.bfloat16):
    """Inputs of the output stage: retention outputs o [B,H,N,dv] ~ N(0,1),
    projection weight [d_out, H*dv] ~ N(0,1)/sqrt(H*dv) (random init, no
    trained weights exist here), GroupNorm weight ~ 1 + 0.1 N(0,1) and bias
    ~ 0.1 N(0,1) (float32 [H*dv]), and a gate ~ U(0,1) [B,N,H*dv]."""
    g = _gen(device, seed)
    K = H * dv
    o = torch.randn((B, H, N, dv), generator=g, device=device, dtype=torch.float32).to(dtype)
    w_o = torch.randn((d_out, K), generator=g, device=device, dtype=torch.float32).mul_(1.0 / math.sqrt(K)).to(dtype)
    gn_w = torch.randn((K,), generator=g, device=device, dtype=torch.float32).mul_(0.1).add_(1.0)
    gn_b = torch.randn((K,), generator=g, device=device, dtype=torch.float32).mul_(0.1)
    gate = torch.rand((B, N, K), generator=g, device=device, dtype=torch.float32).to(dtype)
    return o, w_o, gn_w, gn_b, gate
