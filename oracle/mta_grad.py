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
            depth_scale: float = 1.0, gate: Optional[torch.Tensor] = None, keep: Optional[Dict] = None):
    """float64 forward; every argument a float64 tensor (q, k, v [B,H,T,d],
    theta_kq [H,c_q,c_k], theta_head [H/c_h,c_h,c_h], gn_w/gn_b [H,d], gate [H]).
    With ``keep`` (a dict), the intermediate maps X, C, P, O are stored in it."""
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
    if keep is not None:
        keep.update(X=X, C=C)
    L = C.masked_fill(future, float("-inf"))                  # Mask_-inf
    P = torch.softmax(L, dim=-1)
    Pg = P.reshape(B, G, c_h, T, T)
    P3 = torch.einsum("gab,zgbij->zgaij", theta_head, Pg).reshape(B, H, T, T)  # Eq. 7
    O = torch.matmul(P3, v)
    if keep is not None:
        keep.update(P=P, O=O)
    mu = O.mean(-1, keepdim=True)
    var = ((O - mu) ** 2).mean(-1, keepdim=True)
    Y = (O - mu) / torch.sqrt(var + eps) * gn_w[None, :, None, :] + gn_b[None, :, None, :]
    scale = depth_scale * (torch.sigmoid(gate) if gate is not None else torch.ones(H, dtype=q.dtype))
    return Y * scale[None, :, None, None]


NAMES = ("q", "k", "v", "theta_kq", "theta_head", "gn_w", "gn_b", "gate")


def gradients(inp: Dict[str, torch.Tensor], dout: torch.Tensor, *, c_h: int, exact: bool = False,
              eps: float = 1e-5, depth_scale: float = 1.0, term_scales: bool = False) -> Dict[str, torch.Tensor]:
    """Gradients of sum(dout * forward(inp)) with respect to every input
    (float64; the gate only if ``inp`` has one).

    With ``term_scales``, also "scale_theta_kq" and "scale_theta_head": for the
    two kernel gradients, which are sums over the whole logit map, the sum of
    the magnitudes of their terms down to the products they are built from:
    with M3^a = |dO^a| |V^a|^T (the magnitudes of the terms of dP3^a = dO^a V^aT),
    M^b = sum_a |w_ab| M3^a and DM^b_i = sum_j P^b_ij M^b_ij,
      scale_theta_kq[i'][j'] = sum P (M + DM) |X[i-i'][j-j']|   (dC = P (dP - D)),
      scale_theta_head[a][b] = sum M3^a P^b
    (dO from autograd's gradient with respect to O).  Rounding errors of such
    sums scale with them, also where the exact sum cancels to about zero."""
    leaves = {n: inp[n].detach().double().clone().requires_grad_(True) for n in NAMES if inp.get(n) is not None}
    keep: Dict = {}
    out = forward(leaves["q"], leaves["k"], leaves["v"], leaves["theta_kq"], leaves["theta_head"],
                  leaves["gn_w"], leaves["gn_b"], c_h=c_h, exact=exact, eps=eps, depth_scale=depth_scale,
                  gate=leaves.get("gate"), keep=keep)
    names = list(leaves)
    extra = [keep["O"]] if term_scales else []
    grads = torch.autograd.grad(out, [leaves[n] for n in names] + extra, grad_outputs=dout.double())
    res = dict(zip(names, (g.detach() for g in grads[:len(names)])))
    if term_scales:
        dO = grads[len(names)].detach()
        X, P = keep["X"].detach(), keep["P"].detach()
        v = leaves["v"].detach()
        B, H, T, d = v.shape
        G = H // c_h
        M3 = torch.matmul(dO.abs(), v.abs().transpose(-1, -2))
        wa = leaves["theta_head"].detach().abs()
        M = torch.einsum("gab,zgaij->zgbij", wa, M3.reshape(B, G, c_h, T, T)).reshape(B, H, T, T)
        DM = (P * M).sum(-1, keepdim=True)
        dC_mag = P * (M + DM)
        c_q, c_k = inp["theta_kq"].shape[1], inp["theta_kq"].shape[2]
        idx = torch.arange(T)
        lo = -(c_k // 2)
        sk = torch.zeros((H, c_q, c_k), dtype=torch.float64)
        for ip in range(c_q):
            for jj in range(c_k):
                term = _shift(X, ip, jj + lo).abs()
                if exact:
                    term = term.masked_fill((idx[None, :] - (jj + lo)) > idx[:, None], 0.0)
                sk[:, ip, jj] = (dC_mag * term).sum(dim=(0, 2, 3))
        sw = torch.einsum("zgaij,zgbij->gab", M3.reshape(B, G, c_h, T, T), P.reshape(B, G, c_h, T, T))
        res["scale_theta_kq"] = sk
        res["scale_theta_head"] = sw
    return res
