"""Gradients of the Multi-Token Attention forward: CPU ORACLE (test
infrastructure only; only the tests may import it).

The forward is written again here with plain float64 PyTorch CPU operations,
literally (explicit logit matrix, explicit masks, the key-query convolution as
a sum over its taps of shifted copies of the map, explicit softmax, head mix,
P V, GroupNorm), so that ``torch.autograd`` can differentiate it.  The
gradients come from that library routine; the tests pin them against central
finite differences of the C oracle (``mta_oracle.c``), an independent
implementation of the same function, and pin this forward's values to it.

Placements covered: every one the C oracle has (page "Multi-Token Attention —
Paper Graph", section 3.4): the key-query convolution before the softmax (with
the two-pass masks, or Eq. 4's exact indicator) or after it ("Key-Query
Convolution"), the head mix before or after the softmax ("Head Mixing
Convolution", Eq. 7), both convolutions on one side in the order key-query
first, then heads; GroupNorm with the depth scale and, optionally, the
per-head sigmoid gate ("Group Normalization with Sigmoid Gating").
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


# placement codes, as in the C oracle and the library's configuration
PRE, POST, PRE_EXACT = 0, 1, 2


def _kq_conv(X: torch.Tensor, theta: torch.Tensor, indicator: bool) -> torch.Tensor:
    """Eq. 4 over the last two axes of X [B, H, T, T] with one kernel per head
    (theta [H, c_q, c_k], key offsets -floor(c_k/2) ...): the sum over the taps
    (i', j') of theta[i'][j'] * X[i - i', j - j'], zero padding; with
    ``indicator`` a tap counts only where its key j - j' <= i."""
    T = X.shape[-1]
    c_q, c_k = theta.shape[1], theta.shape[2]
    idx = torch.arange(T)
    lo = -(c_k // 2)
    C = torch.zeros_like(X)
    for ip in range(c_q):
        for jj in range(c_k):
            jp = jj + lo
            term = _shift(X, ip, jp)
            if indicator:
                term = term.masked_fill((idx[None, :] - jp) > idx[:, None], 0.0)
            C = C + theta[None, :, ip, jj, None, None] * term
    return C


def _head_mix(A: torch.Tensor, w: torch.Tensor, c_h: int) -> torch.Tensor:
    """Eq. 7 within each group of c_h heads: out^a = sum_b w[g][a][b] A^b."""
    B, H, T, _ = A.shape
    G = H // c_h
    return torch.einsum("gab,zgbij->zgaij", w, A.reshape(B, G, c_h, T, T)).reshape(B, H, T, T)


def forward(q, k, v, theta_kq, theta_head, gn_w, gn_b, *, c_h: int, exact: bool = False,
            kq_place: Optional[int] = None, head_place: int = POST, eps: float = 1e-5,
            depth_scale: float = 1.0, gate: Optional[torch.Tensor] = None, keep: Optional[Dict] = None):
    """float64 forward; every argument a float64 tensor (q, k, v [B,H,T,d],
    theta_kq [H,c_q,c_k], theta_head [H/c_h,c_h,c_h], gn_w/gn_b [H,d], gate [H]).
    ``kq_place`` PRE / POST / PRE_EXACT (default PRE, or PRE_EXACT when
    ``exact``), ``head_place`` PRE / POST.  With ``keep`` (a dict), the maps
    X (the key-query convolution's input before the softmax), C (its output),
    L (the map entering the softmax), P, P2 (after the convolution that
    follows the softmax), P3 (after the head mix that follows it) and O are
    stored in it."""
    if kq_place is None:
        kq_place = PRE_EXACT if exact else PRE
    B, H, T, d = q.shape
    idx = torch.arange(T)
    future = idx[None, :] > idx[:, None]                      # [i, j]: j > i
    S = torch.matmul(q, k.transpose(-1, -2)) / math.sqrt(d)   # logits, "Standard Multi-Head Attention"
    if kq_place == PRE:                                       # two-pass: Mask_0, then Eq. 4
        X = S.masked_fill(future, 0.0)
        C = _kq_conv(X, theta_kq, False)
    elif kq_place == PRE_EXACT:                               # Eq. 4 with its indicator, on S itself
        X = S
        C = _kq_conv(X, theta_kq, True)
    else:
        X = C = S
    L = _head_mix(C, theta_head, c_h) if head_place == PRE else C
    P = torch.softmax(L.masked_fill(future, float("-inf")), dim=-1)   # Mask_-inf, softmax
    if kq_place == POST:                                      # Eq. 4 on the probabilities, then Mask_0
        P2 = _kq_conv(P, theta_kq, False).masked_fill(future, 0.0)
    else:
        P2 = P
    P3 = _head_mix(P2, theta_head, c_h) if head_place == POST else P2
    O = torch.matmul(P3, v)
    if keep is not None:
        keep.update(X=X, C=C, L=L, P=P, P2=P2, P3=P3, O=O)
    mu = O.mean(-1, keepdim=True)
    var = ((O - mu) ** 2).mean(-1, keepdim=True)
    Y = (O - mu) / torch.sqrt(var + eps) * gn_w[None, :, None, :] + gn_b[None, :, None, :]
    scale = depth_scale * (torch.sigmoid(gate) if gate is not None else torch.ones(H, dtype=q.dtype))
    return Y * scale[None, :, None, None]


NAMES = ("q", "k", "v", "theta_kq", "theta_head", "gn_w", "gn_b", "gate")


def _conv_t_abs(G: torch.Tensor, theta: torch.Tensor) -> torch.Tensor:
    """The transposed convolution with |theta|: y[r][c] = sum over taps of
    |theta[i'][j']| G[r + i'][c + j'] (zero outside [0, T))."""
    c_q, c_k = theta.shape[1], theta.shape[2]
    lo = -(c_k // 2)
    ta = theta.abs()
    y = torch.zeros_like(G)
    for ip in range(c_q):
        for jj in range(c_k):
            y = y + ta[None, :, ip, jj, None, None] * _shift(G, -ip, -(jj + lo))
    return y


def _tap_sums(G: torch.Tensor, X: torch.Tensor, c_q: int, c_k: int, indicator: bool) -> torch.Tensor:
    """[H, c_q, c_k]: sum over batch, i, j of G[i][j] X[i - i'][j - j'] (the
    indicator as in Eq. 4)."""
    B, H, T, _ = G.shape
    idx = torch.arange(T)
    lo = -(c_k // 2)
    s = torch.zeros((H, c_q, c_k), dtype=torch.float64)
    for ip in range(c_q):
        for jj in range(c_k):
            term = _shift(X, ip, jj + lo)
            if indicator:
                term = term.masked_fill((idx[None, :] - (jj + lo)) > idx[:, None], 0.0)
            s[:, ip, jj] = (G * term).sum(dim=(0, 2, 3))
    return s


def _pair_sums(GA: torch.Tensor, XB: torch.Tensor, c_h: int) -> torch.Tensor:
    """[G, c_h, c_h]: [g][a][b] = sum over batch, i, j of GA^a XB^b."""
    B, H, T, _ = GA.shape
    G = H // c_h
    return torch.einsum("zgaij,zgbij->gab", GA.reshape(B, G, c_h, T, T), XB.reshape(B, G, c_h, T, T))


def gradients(inp: Dict[str, torch.Tensor], dout: torch.Tensor, *, c_h: int, exact: bool = False,
              kq_place: Optional[int] = None, head_place: int = POST, eps: float = 1e-5,
              depth_scale: float = 1.0, term_scales: bool = False) -> Dict[str, torch.Tensor]:
    """Gradients of sum(dout * forward(inp)) with respect to every input
    (float64; the gate only if ``inp`` has one).

    With ``term_scales``, also "scale_theta_kq" and "scale_theta_head": for the
    two kernel gradients, which are sums over the whole logit map, the sum of
    the magnitudes of their terms down to the products they are built from.
    Magnitudes are carried backwards through the chain: dP3_mag^a = |dO^a| |V^a|^T
    (the terms of dO^a V^aT); through a head mix, sum_a |w_ab| (.)^a; through
    the convolution after the softmax, the transposed convolution with |theta|
    of the masked map; through the softmax, P (M + sum_j P M) (dC = P (dP - D));
    then
      scale_theta_kq = sum of (magnitude at the convolution's output) x |its input at the tap|,
      scale_theta_head = sum of (magnitude at the mix's output)^a x |its input|^b
    (dO from autograd's gradient with respect to O).  Rounding errors of such
    sums scale with them, also where the exact sum cancels to about zero."""
    if kq_place is None:
        kq_place = PRE_EXACT if exact else PRE
    leaves = {n: inp[n].detach().double().clone().requires_grad_(True) for n in NAMES if inp.get(n) is not None}
    keep: Dict = {}
    out = forward(leaves["q"], leaves["k"], leaves["v"], leaves["theta_kq"], leaves["theta_head"],
                  leaves["gn_w"], leaves["gn_b"], c_h=c_h, kq_place=kq_place, head_place=head_place, eps=eps,
                  depth_scale=depth_scale, gate=leaves.get("gate"), keep=keep)
    names = list(leaves)
    extra = [keep["O"]] if term_scales else []
    grads = torch.autograd.grad(out, [leaves[n] for n in names] + extra, grad_outputs=dout.double())
    res = dict(zip(names, (g.detach() for g in grads[:len(names)])))
    if term_scales:
        dO = grads[len(names)].detach()
        m = {n: t.detach() for n, t in keep.items()}
        v = leaves["v"].detach()
        th = leaves["theta_kq"].detach()
        wa = leaves["theta_head"].detach().abs()
        B, H, T, d = v.shape
        G = H // c_h
        c_q, c_k = th.shape[1], th.shape[2]
        future = torch.arange(T)[None, :] > torch.arange(T)[:, None]

        def mix_t(Mg):  # sum_a |w_ab| Mg^a
            return torch.einsum("gab,zgaij->zgbij", wa, Mg.reshape(B, G, c_h, T, T)).reshape(B, H, T, T)

        M3 = torch.matmul(dO.abs(), v.abs().transpose(-1, -2))
        if head_place == POST:
            res["scale_theta_head"] = _pair_sums(M3, m["P2"].abs(), c_h)
            M2 = mix_t(M3)
        else:
            M2 = M3
        if kq_place == POST:
            M2m = M2.masked_fill(future, 0.0)
            res["scale_theta_kq"] = _tap_sums(M2m, m["P"], c_q, c_k, False)
            M1 = _conv_t_abs(M2m, th)
        else:
            M1 = M2
        P = m["P"]
        ML = P * (M1 + (P * M1).sum(-1, keepdim=True))
        if head_place == PRE:
            res["scale_theta_head"] = _pair_sums(ML, m["C"].abs(), c_h)
            MC = mix_t(ML)
        else:
            MC = ML
        if kq_place != POST:
            res["scale_theta_kq"] = _tap_sums(MC, m["X"].abs(), c_q, c_k, kq_place == PRE_EXACT)
    return res
