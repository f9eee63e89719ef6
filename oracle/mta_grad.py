"""Gradients of the Multi-Token Attention forward: CPU ORACLE (test
infrastructure only; only the tests may import it).

The forward is written again here with plain float64 PyTorch CPU operations,
literally (explicit logit matrix, explicit masks, the key-query convolution as
a sum over its taps of shifted copies of the map, explicit softmax, head mix,
P V, GroupNorm), so that ``torch.autograd`` can differentiate it.  The
gradients come from that library routine; the tests pin them against central
finite differences of the C oracle (``mta_oracle.c``), an independent
implementation of the same function, and pin this forward's values to it.

Placement covered: the key-query convolution before the softmax (two-pass
masks, or Eq. 4's exact indicator) and the head mix after it (page
"Multi-Token Attention — Paper Graph", section 3.4: "Key-Query Convolution",
"Head Mixing Convolution" Eq. 7, "Group Normalization with Sigmoid Gating"),
with the depth scale and, optionally, the per-head sigmoid gate.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import torch


def _shift(x: torch.Tensor, di: int, dj: int) -> torch.Tensor:
    """y[..., i, j] = x[..., i - di, j - dj], zero where the source index is
    outside [0, T) (the convolution's zero padding)."""
    T = x.shape[-1]
    y = torch.zeros_like(x)
    i_lo, i_hi = max(0, di), min(T, T + di)
    j_lo, j_hi = max(0, dj), min(T, T + dj)
    if i_lo < i_hi and j_lo < j_hi:
        y[..., i_lo:i_hi, j_lo:j_hi] = x[..., i_lo - di:i_hi - di, j_lo - dj:j_hi - dj]
    return y


def forward(q, k, v, theta_kq, theta_head, gn_w, gn_b, *, c_h: int, exact: bool = False, eps: float = 1e-5,
            depth_scale: float = 1.0, gate: Optional[torch.Tensor] = None) -> torch.Tensor:
    """float64 forward; every argument a float64 tensor (q, k, v [B,H,T,d],
    theta_kq [H,c_q,c_k], theta_head [H/c_h,c_h,c_h], gn_w/gn_b [H,d], gate [H])."""
    B, H, T, d = q.shape
    c_q, c_k = theta_kq.shape[1], theta_kq.shape[2]
    G = H // c_h
    idx = torch.arange(T)
    future = idx[None, :] > idx[:, None]                      # [i, j]: j > i
    S = torch.matmul(q, k.transpose(-1, -2)) / math.sqrt(d)   # logits, "Standard Multi-Head Attention"
    X = S if exact else S.masked_fill(future, 0.0)            # Mask_0 (two-pass) or the raw map
    C = torch.zeros_like(S)
    lo = -(c_k // 2)
    for ip in range(c_q):                                     # Eq. 4: sum over the taps (i', j')
        for jj in range(c_k):
            jp = jj + lo
            term = _shift(X, ip, jp)                          # X[i - i', j - j']
            if exact:                                         # indicator 1{j - j' <= i}
                term = term.masked_fill((idx[None, :] - jp) > idx[:, None], 0.0)
            C = C + theta_kq[None, :, ip, jj, None, None] * term
    L = C.masked_fill(future, float("-inf"))                  # Mask_-inf
    P = torch.softmax(L, dim=-1)
    Pg = P.reshape(B, G, c_h, T, T)
    P3 = torch.einsum("gab,zgbij->zgaij", theta_head, Pg).reshape(B, H, T, T)  # Eq. 7
    O = torch.matmul(P3, v)
    mu = O.mean(-1, keepdim=True)
    var = ((O - mu) ** 2).mean(-1, keepdim=True)
    Y = (O - mu) / torch.sqrt(var + eps) * gn_w[None, :, None, :] + gn_b[None, :, None, :]
    scale = depth_scale * (torch.sigmoid(gate) if gate is not None else torch.ones(H, dtype=q.dtype))
    return Y * scale[None, :, None, None]


NAMES = ("q", "k", "v", "theta_kq", "theta_head", "gn_w", "gn_b", "gate")


def gradients(inp: Dict[str, torch.Tensor], dout: torch.Tensor, *, c_h: int, exact: bool = False,
              eps: float = 1e-5, depth_scale: float = 1.0) -> Dict[str, torch.Tensor]:
    """Gradients of sum(dout * forward(inp)) with respect to every input
    (float64; the gate only if ``inp`` has one)."""
    leaves = {n: inp[n].detach().double().clone().requires_grad_(True) for n in NAMES if inp.get(n) is not None}
    out = forward(leaves["q"], leaves["k"], leaves["v"], leaves["theta_kq"], leaves["theta_head"],
                  leaves["gn_w"], leaves["gn_b"], c_h=c_h, exact=exact, eps=eps, depth_scale=depth_scale,
                  gate=leaves.get("gate"))
    names = list(leaves)
    grads = torch.autograd.grad(out, [leaves[n] for n in names], grad_outputs=dout.double())
    return dict(zip(names, (g.detach() for g in grads)))
