"""Pins of the CPU oracle against facts the pages and mathematics fix.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with the fact it encodes.  The same
functions run against the real oracle (must all pass) and against builds with
a planted mistake (at least one must fail for each), so the set is shown to
catch a dropped term, a flipped sign or index and a transposed operand.

Facts used (page "Multi-Token Attention — Paper Graph", section 3.4):
  * identity kernels make MTA exactly standard causal attention
    ("Practical Design Choices": identity initialisation) -> library routine
    ``torch.nn.functional.scaled_dot_product_attention`` + ``group_norm``;
  * a key-axis delta one step back is a shift of the keys (the related-work
    note that a one-step key shift is a special case of MTA);
  * the DIFF-Transformer special case of head mixing with weights [1, -lambda]
    ("Head Mixing Convolution");
  * pre-softmax head mixing is a sum of logits, i.e. one attention over
    concatenated features;
  * Eq. 4 written directly over query/key vectors, with the two-pass mask's
    indicator (the input position must not be in its own row's future), and
    with Eq. 4's own indicator (the key must not be in the output row's
    future);
  * softmax rows are distributions over j <= i; causality;
  * hand-derived closed forms in tests/golden/hand_cases.json;
  * brute force at T <= 8 from the definitions;
  * the general layer ("Putting Everything Together"): brute force of the 3D
    and repeated forms, identity kernels give standard attention, a separable
    3D kernel theta3[a][b] = w_ab theta^b is the key-query convolution followed
    by the pre-softmax head mix, and the layer reduces to the single
    placements.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from transformer_attention_variant_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")


def _identity_inputs(cfg):
    inp = I.generate(cfg)
    th = torch.zeros_like(inp["theta_kq"])
    th[:, 0, cfg.c_k // 2] = 1.0
    w = torch.eye(cfg.c_h).expand(cfg.groups, cfg.c_h, cfg.c_h).contiguous()
    inp["theta_kq"], inp["theta_head"] = th, w
    return inp


def _sdpa64(q, k, v, scale=None):
    return F.scaled_dot_product_attention(q.double(), k.double(), v.double(),
                                          is_causal=True, scale=scale)


def _gn64(o, gw, gb, eps, ds):
    """GroupNorm over each head's d channels via torch.nn.functional.group_norm."""
    B, H, T, d = o.shape
    x = o.permute(0, 2, 1, 3).reshape(B * T, H * d)
    y = F.group_norm(x, H, gw.double().reshape(-1), gb.double().reshape(-1), eps)
    return (y.reshape(B, T, H, d).permute(0, 2, 1, 3) * ds)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
def pin_identity_is_causal_attention(lib):
    """Identity kernels: MTA == GroupNorm(SDPA(q,k,v, causal)) x depth scale,
    for every placement of the two convolutions, ragged T and c_h in {1,2,4}."""
    for (kq, hd, ch, T, cq, ck) in [(I.PRE, I.POST, 2, 37, 3, 5), (I.POST, I.POST, 2, 29, 2, 3),
                                    (I.PRE, I.PRE, 4, 23, 4, 4), (I.POST, I.PRE, 1, 19, 3, 7),
                                    (I.PRE_EXACT, I.POST, 2, 31, 3, 6)]:
        cfg = I.small(B=2, H=4, T=T, d=8, c_q=cq, c_k=ck, c_h=ch, kq_place=kq,
                      head_place=hd, gn_random=True, layer=3, seed=11 + T)
        inp = _identity_inputs(cfg)
        got = oracle.forward_cfg(cfg, inp, lib=lib, threads=2)
        ref = _gn64(_sdpa64(inp["q"], inp["k"], inp["v"]), inp["gn_w"], inp["gn_b"],
                    cfg.gn_eps, cfg.depth_scale)
        _close(got, ref.numpy(), 1e-10, f"identity {cfg.short()}")


def pin_sigmoid_gate(lib):
    """Sigmoid-gated GroupNorm ("Group Normalization with Sigmoid Gating"): with
    identity kernels, head h's output is GroupNorm(SDPA) x sigmoid(g_h) x depth
    scale, computed with torch.sigmoid and group_norm."""
    for kq in (I.PRE, I.POST):
        cfg = I.small(B=2, H=4, T=29, d=8, c_q=3, c_k=5, c_h=2, kq_place=kq, gn_random=True,
                      gated=True, layer=2, seed=61)
        inp = _identity_inputs(cfg)
        got = oracle.forward_cfg(cfg, inp, lib=lib, threads=2)
        ref = _gn64(_sdpa64(inp["q"], inp["k"], inp["v"]), inp["gn_w"], inp["gn_b"], cfg.gn_eps,
                    cfg.depth_scale)
        ref = ref * torch.sigmoid(inp["gate"].double())[None, :, None, None]
        _close(got, ref.numpy(), 1e-10, f"gate {cfg.short()}")


def pin_key_shift_is_shifted_attention(lib):
    """A key-axis delta at j' = +1 reads key j-1: MTA == SDPA with the keys
    shifted down one step (k'_j = k_{j-1}, k'_0 = 0); Mask_0 has no effect
    because j-1 <= i whenever j <= i."""
    cfg = I.small(B=1, H=2, T=21, d=8, c_q=2, c_k=5, c_h=1, kq_place=I.PRE, seed=5)
    inp = _identity_inputs(cfg)
    th = torch.zeros_like(inp["theta_kq"])
    th[:, 0, cfg.c_k // 2 + 1] = 1.0          # j' = +1
    inp["theta_kq"] = th
    got = oracle.stages_cfg(cfg, inp, lib=lib, b=0, g=1)["O"][0]
    k = inp["k"].double()
    ks = torch.zeros_like(k)
    ks[:, :, 1:] = k[:, :, :-1]
    ref = _sdpa64(inp["q"], ks, inp["v"])[0, 1]
    _close(got, ref.numpy(), 1e-12, "key shift")


def pin_diff_transformer_special_case(lib):
    """c_h = 2, w = [[1, -lam], [0, 1]], identity key-query kernel, post-softmax
    mix: O^0 = SDPA(q0,k0,v0) - lam SDPA(q1,k1,v0), O^1 = SDPA(q1,k1,v1)."""
    lam = 0.375  # exactly representable in fp32, the kernel tensors' dtype
    cfg = I.small(B=1, H=2, T=25, d=8, c_q=1, c_k=1, c_h=2, seed=9)
    inp = _identity_inputs(cfg)
    inp["theta_head"] = torch.tensor([[[1.0, -lam], [0.0, 1.0]]])
    O = oracle.stages_cfg(cfg, inp, lib=lib)["O"]
    q, k, v = inp["q"][0], inp["k"][0], inp["v"][0]
    a00 = _sdpa64(q[0:1], k[0:1], v[0:1])[0]
    a10 = _sdpa64(q[1:2], k[1:2], v[0:1])[0]
    a11 = _sdpa64(q[1:2], k[1:2], v[1:2])[0]
    _close(O[0], (a00 - lam * a10).numpy(), 1e-12, "DIFF head 0")
    _close(O[1], a11.numpy(), 1e-12, "DIFF head 1")


def pin_pre_softmax_head_mix_is_concat_attention(lib):
    """Pre-softmax mixing adds logits: w00 S^0 + w01 S^1 = [w00 q0, w01 q1].[k0, k1]
    / sqrt(d), i.e. SDPA over concatenated features with scale 1/sqrt(d)."""
    cfg = I.small(B=1, H=2, T=23, d=8, c_q=1, c_k=1, c_h=2, head_place=I.PRE, seed=13)
    inp = _identity_inputs(cfg)
    w = torch.tensor([[[0.9, 0.4], [-0.3, 1.1]]])
    inp["theta_head"] = w
    O = oracle.stages_cfg(cfg, inp, lib=lib)["O"]
    q, k, v = inp["q"][0].double(), inp["k"][0].double(), inp["v"][0].double()
    for a in range(2):
        qc = torch.cat([w[0, a, 0] * q[0], w[0, a, 1] * q[1]], dim=-1)[None]
        kc = torch.cat([k[0], k[1]], dim=-1)[None]
        ref = _sdpa64(qc, kc, v[a:a + 1], scale=1.0 / math.sqrt(cfg.d))[0]
        _close(O[a], ref.numpy(), 1e-12, f"pre-softmax mix head {a}")


def _eq4_two_pass(q, k, theta, i, j, d):
    """Eq. 4 summed over vectors, with the two-pass indicator: tap (i',j')
    contributes theta q_{i-i'} . k_{j-j'} / sqrt(d) iff both indices are >= 0
    and the key is not in the future of its own query row (j-j' <= i-i')."""
    c_q, c_k = theta.shape
    tot = 0.0
    for ip in range(c_q):
        for jp in range(-(c_k // 2), (c_k + 1) // 2):
            a, bb = i - ip, j - jp
            if a < 0 or bb < 0 or bb > a:
                continue
            tot += theta[ip, jp + c_k // 2] * float(np.dot(q[a], k[bb])) / math.sqrt(d)
    return tot


def _eq4_exact(q, k, theta, i, j, d):
    """Eq. 4 summed over vectors with its own indicator 1{i >= j-j'}: tap
    (i',j') contributes iff both indices are >= 0 and the key is not in the
    future of the output query i."""
    c_q, c_k = theta.shape
    tot = 0.0
    for ip in range(c_q):
        for jp in range(-(c_k // 2), (c_k + 1) // 2):
            a, bb = i - ip, j - jp
            if a < 0 or bb < 0 or bb > i:
                continue
            tot += theta[ip, jp + c_k // 2] * float(np.dot(q[a], k[bb])) / math.sqrt(d)
    return tot


def pin_eq4_exact_indicator(lib):
    """The exact form: the convolved logit map equals Eq. 4 with its indicator,
    evaluated on query/key vectors at every causal (i, j); it differs from the
    two-pass map on the diagonal band and equals it off the band.  Random
    asymmetric kernel, odd and even c_k, c_q > 1."""
    for (cq, ck, T) in [(3, 5, 19), (4, 4, 15)]:
        cfg = I.small(B=1, H=2, T=T, d=4, c_q=cq, c_k=ck, c_h=2, theta_std=0.7, seed=41 + ck,
                      kq_place=I.PRE_EXACT)
        inp = I.generate(cfg)
        C = oracle.stages_cfg(cfg, inp, lib=lib)["C"]
        C2 = oracle.stages_cfg(I.with_(cfg, kq_place=I.PRE), inp, lib=lib)["C"]
        q = inp["q"].double().numpy()[0]
        k = inp["k"].double().numpy()[0]
        th = inp["theta_kq"].double().numpy()
        band = cq - 1 + ck // 2
        for h in range(2):
            for i in range(T):
                for j in range(i + 1):
                    ref = _eq4_exact(q[h], k[h], th[h], i, j, cfg.d)
                    assert abs(C[h, i, j] - ref) <= 1e-12, ("eq4 exact", cq, ck, h, i, j, C[h, i, j], ref)
                    if j < i - band + 1:
                        assert abs(C[h, i, j] - C2[h, i, j]) <= 1e-12, ("off-band", i, j)
            assert np.max(np.abs(C[h] - C2[h])) > 1e-3, "the two forms must differ on the band"


def pin_eq4_vector_form(lib):
    """The convolved logit map (kq pre-softmax) equals Eq. 4 evaluated directly on
    query/key vectors with the two-pass indicator, at every causal (i, j); off
    the diagonal band it equals Eq. 4 with no mask at all.  Random asymmetric
    kernel, odd and even c_k."""
    for (cq, ck, T) in [(3, 5, 19), (2, 4, 15)]:
        cfg = I.small(B=1, H=2, T=T, d=4, c_q=cq, c_k=ck, c_h=2, theta_std=0.7, seed=17 + ck)
        inp = I.generate(cfg)
        C = oracle.stages_cfg(cfg, inp, lib=lib)["C"]
        q = inp["q"].double().numpy()[0]
        k = inp["k"].double().numpy()[0]
        th = inp["theta_kq"].double().numpy()
        for h in range(2):
            for i in range(T):
                for j in range(i + 1):
                    ref = _eq4_two_pass(q[h], k[h], th[h], i, j, cfg.d)
                    assert abs(C[h, i, j] - ref) <= 1e-12, ("eq4", cq, ck, h, i, j, C[h, i, j], ref)
            # off-band: no tap is masked, so the plain Eq. 4 sum holds
            i, j = T - 1, 1
            assert j + ck // 2 <= i - cq + 1
            full = 0.0
            for ip in range(cq):
                for jp in range(-(ck // 2), (ck + 1) // 2):
                    if j - jp >= 0:
                        full += th[h, ip, jp + ck // 2] * float(np.dot(q[h, i - ip], k[h, j - jp])) / math.sqrt(cfg.d)
            assert abs(C[h, i, j] - full) <= 1e-12


def pin_softmax_rows_are_distributions(lib):
    """Rows of P sum to 1 and vanish in the future; with a post-softmax head
    mix the rows of P3^a sum to sum_b w_ab; post-softmax key-query conv leaves
    the future exactly 0 (its final Mask_0)."""
    for kq in (I.PRE, I.POST):
        cfg = I.small(B=1, H=4, T=31, d=8, c_q=3, c_k=5, c_h=2, kq_place=kq, seed=19)
        inp = I.generate(cfg)
        st = oracle.stages_cfg(cfg, inp, lib=lib, g=1)
        P, P2, P3 = st["P"], st["P2"], st["P3"]
        fut = np.triu(np.ones((cfg.T, cfg.T), dtype=bool), 1)
        assert np.all(P[:, fut] == 0.0) and np.all(P2[:, fut] == 0.0)
        _close(P.sum(-1), np.ones((2, cfg.T)), 1e-12, "row sums")
        assert np.all(P[:, ~fut] > 0.0)
        if kq == I.PRE:
            w = inp["theta_head"][1].double().numpy()
            _close(P3.sum(-1), np.repeat(w.sum(1)[:, None], cfg.T, 1), 1e-12, "mixed row sums")


def pin_causality(lib):
    """Changing q, k, v at positions > t leaves out[..., :t+1, :] bitwise equal."""
    for (kq, hd) in [(I.PRE, I.POST), (I.POST, I.POST), (I.PRE, I.PRE), (I.POST, I.PRE),
                     (I.PRE_EXACT, I.POST)]:
        cfg = I.small(B=1, H=4, T=33, d=8, c_q=4, c_k=7, c_h=2, kq_place=kq, head_place=hd, seed=23)
        inp = I.generate(cfg)
        base = oracle.forward_cfg(cfg, inp, lib=lib, threads=2)
        t = 17
        g = torch.Generator().manual_seed(3)
        for name in ("q", "k", "v"):
            pert = dict(inp)
            x = pert[name].clone()
            x[:, :, t + 1:] += torch.randn(x[:, :, t + 1:].shape, generator=g) * 5
            pert[name] = x
            o2 = oracle.forward_cfg(cfg, pert, lib=lib, threads=2)
            assert np.array_equal(base[:, :, :t + 1], o2[:, :, :t + 1]), (kq, hd, name)
            assert not np.array_equal(base[:, :, t + 1:], o2[:, :, t + 1:])


def pin_hand_cases(lib):
    """Hand-derived closed forms (tests/golden/hand_cases.json)."""
    cases = json.load(open(GOLDEN))["cases"]
    for cs in cases:
        T, ch = cs["T"], cs["c_h"]
        shp = (1, ch, T, 1)
        q = torch.tensor(cs["q"], dtype=torch.float64).reshape(shp)
        k = torch.tensor(cs["k"], dtype=torch.float64).reshape(shp)
        v = torch.tensor(cs["v"], dtype=torch.float64).reshape(shp)
        th = torch.tensor(cs["theta_kq"], dtype=torch.float64).reshape(ch, cs["c_q"], cs["c_k"])
        w = torch.tensor(cs["theta_head"], dtype=torch.float64).reshape(1, ch, ch)
        st = oracle.stages(q, k, v, th, w, torch.ones(ch, 1), torch.zeros(ch, 1),
                           c_q=cs["c_q"], c_k=cs["c_k"], c_h=ch, kq_place=cs["kq_place"],
                           head_place=cs["head_place"], lib=lib)
        exp = cs["expected_O"]
        if ch == 1:
            exp = [exp]
        for a in range(ch):
            for t in range(T):
                e = eval(exp[a][t], {"math": math})
                assert abs(st["O"][a, t, 0] - e) <= 1e-12, (cs["name"], a, t, st["O"][a, t, 0], e)


def _brute(q, k, v, th, w, gw, gb, c_q, c_k, c_h, kq, hd, eps, ds):
    """Brute force from the definitions, one scalar at a time (T <= 8)."""
    B, H, T, d = q.shape
    out = np.zeros_like(q)
    lo, hi = -(c_k // 2), (c_k + 1) // 2 - 1

    def conv(Xh, h, i, j, exact=False):
        s = 0.0
        for ip in range(c_q):
            for jp in range(lo, hi + 1):
                a, bb = i - ip, j - jp
                if 0 <= a < T and 0 <= bb < T and (bb <= i or not exact):
                    s += th[h, ip, jp - lo] * Xh[a][bb]
        return s

    for b in range(B):
        for g in range(H // c_h):
            hs = list(range(g * c_h, (g + 1) * c_h))
            S = {h: [[float(np.dot(q[b, h, a], k[b, h, j])) / math.sqrt(d) for j in range(T)]
                     for a in range(T)] for h in hs}
            if kq == I.PRE:
                M0 = {h: [[S[h][a][j] if j <= a else 0.0 for j in range(T)] for a in range(T)] for h in hs}
                L = {h: [[conv(M0[h], h, i, j) for j in range(T)] for i in range(T)] for h in hs}
            elif kq == I.PRE_EXACT:
                L = {h: [[conv(S[h], h, i, j, exact=True) for j in range(T)] for i in range(T)] for h in hs}
            else:
                L = S
            if hd == I.PRE:
                L = {hs[x]: [[sum(w[g, x, y] * L[hs[y]][i][j] for y in range(c_h)) for j in range(T)]
                             for i in range(T)] for x in range(c_h)}
            P = {}
            for h in hs:
                P[h] = []
                for i in range(T):
                    row = [L[h][i][j] for j in range(i + 1)]
                    m = max(row)
                    e = [math.exp(x - m) for x in row]
                    s = sum(e)
                    P[h].append([x / s for x in e] + [0.0] * (T - i - 1))
            if kq == I.POST:
                P = {h: [[conv(P[h], h, i, j) if j <= i else 0.0 for j in range(T)] for i in range(T)]
                     for h in hs}
            if hd == I.POST:
                P = {hs[x]: [[sum(w[g, x, y] * P[hs[y]][i][j] for y in range(c_h)) for j in range(T)]
                             for i in range(T)] for x in range(c_h)}
            for h in hs:
                for i in range(T):
                    o = [sum(P[h][i][j] * v[b, h, j, c] for j in range(T)) for c in range(d)]
                    mu = sum(o) / d
                    var = sum((x - mu) ** 2 for x in o) / d
                    for c in range(d):
                        out[b, h, i, c] = ((o[c] - mu) / math.sqrt(var + eps) * gw[h, c] + gb[h, c]) * ds
    return out


def pin_brute_force_tiny(lib):
    """Whole pipeline vs scalar brute force, all four placements, T <= 8,
    c_q > T, even c_k."""
    for (kq, hd, T, cq, ck, ch) in [(I.PRE, I.POST, 8, 3, 5, 2), (I.POST, I.POST, 7, 2, 3, 2),
                                    (I.PRE, I.PRE, 6, 9, 4, 2), (I.POST, I.PRE, 5, 3, 6, 4),
                                    (I.PRE, I.POST, 1, 2, 3, 1), (I.PRE_EXACT, I.POST, 8, 3, 5, 2),
                                    (I.PRE_EXACT, I.PRE, 6, 9, 4, 2), (I.PRE, I.POST, 5, 2, 3, 8)]:
        cfg = I.small(B=2, H=max(4, ch), T=T, d=4, c_q=cq, c_k=ck, c_h=ch, kq_place=kq, head_place=hd,
                      theta_std=0.5, head_std=0.5, gn_random=True, layer=2, seed=31 + T)
        inp = I.generate(cfg)
        got = oracle.forward_cfg(cfg, inp, lib=lib, threads=1)
        n = {kk: t.double().numpy() for kk, t in inp.items()}
        ref = _brute(n["q"], n["k"], n["v"], n["theta_kq"], n["theta_head"], n["gn_w"], n["gn_b"],
                     cq, ck, ch, kq, hd, cfg.gn_eps, cfg.depth_scale)
        _close(got, ref, 1e-10, f"brute {cfg.short()}")


def _brute_layer(q, k, v, gw, gb, eps, ds, c_q, c_k, c_h, exact=False, kq_pre=None, head_pre=None,
                 conv3d=None, head_post=None, kq_post=None, head_post2=None, c_q2=0, c_k2=0):
    """The general layer, one scalar at a time from the definitions (T <= 8)."""
    B, H, T, d = q.shape
    out = np.zeros_like(q)

    def conv(X, th, cq, ck, i, j, ind):
        lo = -(ck // 2)
        s = 0.0
        for ip in range(cq):
            for jp in range(lo, lo + ck):
                a, bb = i - ip, j - jp
                if 0 <= a < T and 0 <= bb < T and (not ind or bb <= i):
                    s += th[ip, jp - lo] * X[a][bb]
        return s

    def mix(M, w, rows):
        return [[[sum(w[x, y] * M[y][i][j] for y in range(c_h)) for j in range(T)] for i in range(T)]
                for x in range(c_h)]

    for b in range(B):
        for g in range(H // c_h):
            hs = list(range(g * c_h, (g + 1) * c_h))
            S = [[[float(np.dot(q[b, h, i], k[b, h, j])) / math.sqrt(d) for j in range(T)] for i in range(T)]
                 for h in hs]
            M0 = [[[S[x][i][j] if (exact or j <= i) else 0.0 for j in range(T)] for i in range(T)]
                  for x in range(c_h)]
            if conv3d is not None:
                L = [[[sum(conv(M0[y], conv3d[g, x, y], c_q, c_k, i, j, exact) for y in range(c_h))
                       for j in range(T)] for i in range(T)] for x in range(c_h)]
            elif kq_pre is not None:
                L = [[[conv(M0[x], kq_pre[hs[x]], c_q, c_k, i, j, exact) for j in range(T)] for i in range(T)]
                     for x in range(c_h)]
            else:
                L = S
            if head_pre is not None and conv3d is None:
                L = mix(L, head_pre[g], T)
            P = []
            for x in range(c_h):
                rows = []
                for i in range(T):
                    r = [L[x][i][j] for j in range(i + 1)]
                    m = max(r)
                    e = [math.exp(t - m) for t in r]
                    z = sum(e)
                    rows.append([t / z for t in e] + [0.0] * (T - i - 1))
                P.append(rows)
            if head_post is not None:
                P = mix(P, head_post[g], T)
            if kq_post is not None:
                P = [[[conv(P[x], kq_post[hs[x]], c_q2, c_k2, i, j, False) if j <= i else 0.0
                       for j in range(T)] for i in range(T)] for x in range(c_h)]
            if head_post2 is not None:
                P = mix(P, head_post2[g], T)
            for x, h in enumerate(hs):
                for i in range(T):
                    o = [sum(P[x][i][j] * v[b, h, j, c] for j in range(T)) for c in range(d)]
                    mu = sum(o) / d
                    var = sum((t - mu) ** 2 for t in o) / d
                    for c in range(d):
                        out[b, h, i, c] = ((o[c] - mu) / math.sqrt(var + eps) * gw[h, c] + gb[h, c]) * ds
    return out


def _layer_inputs(cfg):
    inp = I.generate(cfg)
    n = {kk: t.double().numpy() for kk, t in inp.items()}
    w = {kk: (vv.double().numpy() if hasattr(vv, "double") else vv)
         for kk, vv in I.layer_weights(cfg, inp).items()}
    return inp, n, w


def pin_layer_brute_force(lib):
    """The 3D-convolution and repeated forms (and a layer with every stage
    present) against scalar brute force, T <= 8, c_q larger than T, even c_k."""
    cases = [
        I.small(B=1, H=4, T=7, d=4, c_q=3, c_k=4, c_h=2, form="3d", head_place=I.PRE, theta_std=0.5,
                gn_random=True, layer=2, seed=91),
        I.small(B=1, H=4, T=6, d=4, c_q=2, c_k=3, c_h=4, form="3d", kq_place=I.PRE_EXACT, head_place=I.PRE,
                theta_std=0.5, seed=92),
        I.small(B=2, H=4, T=8, d=4, c_q=3, c_k=5, c_h=2, form="repeat", c_q2=2, c_k2=4, theta_std=0.4,
                head_std=0.4, gn_random=True, seed=93),
        I.small(B=1, H=2, T=5, d=4, c_q=9, c_k=3, c_h=1, form="repeat", c_q2=3, c_k2=3,
                kq_place=I.PRE_EXACT, theta_std=0.4, seed=94),
    ]
    for cfg in cases:
        inp, n, w = _layer_inputs(cfg)
        got = oracle.layer(inp["q"], inp["k"], inp["v"], inp["gn_w"], inp["gn_b"], c_q=cfg.c_q, c_k=cfg.c_k,
                           c_h=cfg.c_h, eps=cfg.gn_eps, depth_scale=cfg.depth_scale, lib=lib, threads=1,
                           **I.layer_weights(cfg, inp))
        ref = _brute_layer(n["q"], n["k"], n["v"], n["gn_w"], n["gn_b"], cfg.gn_eps, cfg.depth_scale,
                           cfg.c_q, cfg.c_k, cfg.c_h, **w)
        _close(got, ref, 1e-10, f"layer brute {cfg.short()}")
    # every stage at once (3D excluded: it replaces the pre-softmax pair)
    cfg = I.small(B=1, H=4, T=7, d=4, c_q=2, c_k=3, c_h=2, form="repeat", c_q2=3, c_k2=2, theta_std=0.4,
                  head_std=0.4, seed=95)
    inp, n, w = _layer_inputs(cfg)
    extra = (torch.randn((2, 2, 2), generator=torch.Generator().manual_seed(7)) * 0.4 + torch.eye(2)).double()
    got = oracle.layer(inp["q"], inp["k"], inp["v"], inp["gn_w"], inp["gn_b"], c_q=cfg.c_q, c_k=cfg.c_k,
                       c_h=cfg.c_h, eps=cfg.gn_eps, depth_scale=cfg.depth_scale, lib=lib, threads=1,
                       head_pre=extra, **I.layer_weights(cfg, inp))
    ref = _brute_layer(n["q"], n["k"], n["v"], n["gn_w"], n["gn_b"], cfg.gn_eps, cfg.depth_scale,
                       cfg.c_q, cfg.c_k, cfg.c_h, head_pre=extra.numpy(), **w)
    _close(got, ref, 1e-10, "layer brute, all stages")


def pin_layer_identity_is_attention(lib):
    """Identity kernels in every stage of the repeated form, and an identity
    3D kernel, give standard causal attention (library routine)."""
    for form in ("repeat", "3d"):
        cfg = I.small(B=2, H=4, T=23, d=8, c_q=3, c_k=5, c_h=2, form=form, c_q2=2, c_k2=3,
                      head_place=I.PRE if form == "3d" else I.POST, gn_random=True, seed=97)
        inp = I.generate(cfg)
        w = I.layer_weights(cfg, inp)
        for name in ("kq_pre", "kq_post"):
            if name in w:
                t = torch.zeros_like(w[name])
                t[:, 0, t.shape[2] // 2] = 1.0
                w[name] = t
        for name in ("head_post", "head_post2"):
            if name in w:
                w[name] = torch.eye(cfg.c_h).expand(cfg.groups, cfg.c_h, cfg.c_h).contiguous()
        if "conv3d" in w:
            t = torch.zeros_like(w["conv3d"])
            for a in range(cfg.c_h):
                t[:, a, a, 0, cfg.c_k // 2] = 1.0
            w["conv3d"] = t
        got = oracle.layer(inp["q"], inp["k"], inp["v"], inp["gn_w"], inp["gn_b"], c_q=cfg.c_q, c_k=cfg.c_k,
                           c_h=cfg.c_h, eps=cfg.gn_eps, depth_scale=cfg.depth_scale, lib=lib, threads=2, **w)
        ref = _gn64(_sdpa64(inp["q"], inp["k"], inp["v"]), inp["gn_w"], inp["gn_b"], cfg.gn_eps,
                    cfg.depth_scale)
        _close(got, ref.numpy(), 1e-10, f"layer identity {form}")


def pin_layer_separable_3d(lib):
    """A separable 3D kernel theta3[a][b] = w_ab theta^b is the key-query
    convolution of each head followed by the pre-softmax head mix (linearity),
    and the layer with one key-query and one head stage equals every single
    placement of the two convolutions."""
    cfg = I.small(B=1, H=4, T=19, d=8, c_q=3, c_k=5, c_h=2, kq_place=I.PRE, head_place=I.PRE,
                  theta_std=0.3, head_std=0.3, seed=98)
    inp = I.generate(cfg)
    th, w = inp["theta_kq"].double(), inp["theta_head"].double()
    G, ch = cfg.groups, cfg.c_h
    t3 = torch.zeros((G, ch, ch, cfg.c_q, cfg.c_k), dtype=torch.float64)
    for g in range(G):
        for a in range(ch):
            for b in range(ch):
                t3[g, a, b] = w[g, a, b] * th[g * ch + b]
    for exact in (False, True):
        got = oracle.layer(inp["q"], inp["k"], inp["v"], inp["gn_w"], inp["gn_b"], c_q=cfg.c_q, c_k=cfg.c_k,
                           c_h=ch, eps=cfg.gn_eps, depth_scale=cfg.depth_scale, conv3d=t3, exact=exact,
                           lib=lib, threads=2)
        ref = oracle.forward(inp["q"], inp["k"], inp["v"], th, w, inp["gn_w"], inp["gn_b"], c_q=cfg.c_q,
                             c_k=cfg.c_k, c_h=ch, kq_place=I.PRE_EXACT if exact else I.PRE,
                             head_place=I.PRE, eps=cfg.gn_eps, depth_scale=cfg.depth_scale, lib=lib,
                             threads=2)
        _close(got, ref, 1e-11, f"separable 3D exact={exact}")
    for kq in (I.PRE, I.POST, I.PRE_EXACT):
        for hd in (I.PRE, I.POST):
            c2 = I.with_(cfg, kq_place=kq, head_place=hd)
            got = oracle.layer(inp["q"], inp["k"], inp["v"], inp["gn_w"], inp["gn_b"], c_q=cfg.c_q,
                               c_k=cfg.c_k, c_h=ch, eps=cfg.gn_eps, depth_scale=cfg.depth_scale, lib=lib,
                               threads=2, **I.layer_weights(c2, inp))
            ref = oracle.forward_cfg(c2, inp, lib=lib, threads=2)
            _close(got, ref, 1e-12, f"layer = placement {c2.short()}")


def pin_layer_causality(lib):
    """Changing q, k, v after position t leaves the layer's output up to t
    bitwise unchanged (3D and repeated forms)."""
    for form in ("3d", "repeat"):
        cfg = I.small(B=1, H=4, T=29, d=8, c_q=4, c_k=7, c_h=2, form=form, c_q2=3, c_k2=5,
                      head_place=I.PRE if form == "3d" else I.POST, seed=99)
        inp = I.generate(cfg)
        base = oracle.forward_cfg(cfg, inp, lib=lib, threads=2)
        t = 13
        gen = torch.Generator().manual_seed(4)
        for name in ("q", "k", "v"):
            pert = dict(inp)
            x = pert[name].clone()
            x[:, :, t + 1:] += torch.randn(x[:, :, t + 1:].shape, generator=gen) * 5
            pert[name] = x
            o2 = oracle.forward_cfg(cfg, pert, lib=lib, threads=2)
            assert np.array_equal(base[:, :, :t + 1], o2[:, :, :t + 1]), (form, name)
            assert not np.array_equal(base[:, :, t + 1:], o2[:, :, t + 1:])


def pin_head_permutation_large_groups(lib):
    """Groups of 8 and 16 heads (the page's default c_h is 16): with the
    identity key-query kernel and a permutation pi as each group's mixing
    matrix after the softmax, Eq. 7 hands head a the probabilities of head
    pi(a), so O^a = softmax(Q^pi(a) K^pi(a)^T / sqrt(d)) V^a: causal attention
    with the queries and keys of head pi(a) and the values of head a."""
    for (ch, H, T) in ((8, 8, 27), (16, 16, 21)):
        cfg = I.small(B=2, H=H, T=T, d=8, c_q=3, c_k=5, c_h=ch, gn_random=True, layer=2, seed=51 + ch)
        inp = _identity_inputs(cfg)
        g = torch.Generator().manual_seed(ch)
        w = torch.zeros(cfg.groups, ch, ch, dtype=torch.float32)
        perm = []
        for grp in range(cfg.groups):
            pi = torch.randperm(ch, generator=g)
            w[grp, torch.arange(ch), pi] = 1.0
            perm += [grp * ch + int(x) for x in pi]
        inp["theta_head"] = w
        got = oracle.forward_cfg(cfg, inp, lib=lib, threads=2)
        src = torch.tensor(perm)
        o = _sdpa64(inp["q"][:, src], inp["k"][:, src], inp["v"])
        ref = _gn64(o, inp["gn_w"], inp["gn_b"], cfg.gn_eps, cfg.depth_scale)
        _close(got, ref.numpy(), 1e-10, f"head permutation {cfg.short()}")


ALL_PINS = [
    pin_identity_is_causal_attention,
    pin_sigmoid_gate,
    pin_key_shift_is_shifted_attention,
    pin_diff_transformer_special_case,
    pin_pre_softmax_head_mix_is_concat_attention,
    pin_eq4_vector_form,
    pin_eq4_exact_indicator,
    pin_softmax_rows_are_distributions,
    pin_causality,
    pin_hand_cases,
    pin_brute_force_tiny,
    pin_head_permutation_large_groups,
    pin_layer_brute_force,
    pin_layer_identity_is_attention,
    pin_layer_separable_3d,
    pin_layer_causality,
]
