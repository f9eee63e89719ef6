"""Seeded synthetic inputs for the Multi-Token Attention forward.

This module only draws random numbers and lays out buffers; it holds none of
the method's arithmetic.  It is the one piece shared by the GPU path's tests
and benchmark and by the CPU oracle's tests.

The workloads stand in for the ones on the page "Multi-Token Attention —
Paper Graph": the toy block-location task (section 4.1 / Table 1: c_q = L = 2
query letters, c_k = 2N-1 = 9 for N = 5), the 880M-parameter model's attention
layer ("Training configuration": 16 heads, context 2048), its 4K-context
finetune with multi-needle retrieval (Figure 3), and a sweep over the kernel
sizes of the Table 5 ablations.  No dataset or trained weight is used: every
tensor is drawn from a seeded ``torch.Generator``.

Kernels are "identity plus noise": the key-query kernel is a delta at
(i'=0, j'=0), stored at column floor(c_k/2), and each head-mixing block is the
identity ("Practical Design Choices": identity initialisation), with Gaussian
noise added to every entry.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict, List

import torch

PRE = 0
POST = 1
PRE_EXACT = 2   # key-query convolution before the softmax with Eq. 4's exact indicator
F32 = 0
BF16 = 1

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class MTAConfig:
    name: str
    B: int
    H: int
    T: int
    d: int
    c_q: int
    c_k: int
    c_h: int
    kq_place: int = PRE
    head_place: int = POST
    dtype: str = "bf16"
    qkv_std: float = 1.0
    theta_std: float = 0.05
    head_std: float = 0.05
    layer: int = 1
    needles: int = 0
    needle_queries: int = 32
    needle_scale: float = 3.0  # needle keys are needle_scale x the direction u
    # False: a needle key is replaced by needle_scale * u (all needles of a row
    # give the same logit); True: needle_scale * u is added to the key's own
    # draw, so the needles of a row compete with logits a few units apart
    needle_on_key: bool = False
    seed: int = 0
    gn_eps: float = 1e-5
    gn_random: bool = False
    gated: bool = False   # per-head sigmoid gate on the GroupNorm output
    gate_std: float = 1.0  # spread of the gate logits g_h ~ N(0, gate_std^2)
    # "std": one key-query and one head convolution, placed by kq_place / head_place;
    # "3d": the both-pre-softmax 3D convolution (kernel [G][c_h][c_h][c_q][c_k]);
    # "repeat": kq conv before the softmax, head mix after it, then a second
    #   key-query (c_q2 x c_k2) and head convolution after the softmax
    form: str = "std"
    c_q2: int = 0
    c_k2: int = 0

    @property
    def depth_scale(self) -> float:
        # the layer-dependent depth scale: 1 / sqrt(layer) (1 for layer 1)
        return 1.0 / math.sqrt(self.layer)

    @property
    def groups(self) -> int:
        return self.H // self.c_h

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def causal_logits(self) -> int:
        """Causal (query, key) pairs over all heads: B*H*T(T+1)/2."""
        return self.B * self.H * self.T * (self.T + 1) // 2

    def alg_flops(self) -> Dict[str, float]:
        """Algorithmic FLOP, each causal logit counted once: QK^T and PV on the
        matrix cores (4d), the key-query stencil (2 c_q c_k) and the head mix
        (2 c_h) on the vector ALUs."""
        n = float(self.causal_logits())
        if self.form == "3d":      # c_h source kernels per output head, no separate mix
            return {"contraction": n * 4 * self.d, "stencil": n * 2 * self.c_q * self.c_k * self.c_h,
                    "mix": 0.0}
        if self.form == "repeat":  # two key-query and two head convolutions
            return {"contraction": n * 4 * self.d,
                    "stencil": n * 2 * (self.c_q * self.c_k + self.c_q2 * self.c_k2),
                    "mix": n * 4 * self.c_h}
        return {
            "contraction": n * 4 * self.d,
            "stencil": n * 2 * self.c_q * self.c_k,
            "mix": n * 2 * self.c_h,
        }

    def io_bytes(self) -> int:
        """Compulsory HBM bytes of one call: read q, k, v, write out."""
        el = 4 if self.dtype == "f32" else 2
        return 4 * self.B * self.H * self.T * self.d * el

    def short(self) -> str:
        kq = {PRE: "pre", POST: "post", PRE_EXACT: "exact"}[self.kq_place]
        hd = "pre" if self.head_place == PRE else "post"
        form = "" if self.form == "std" else f"_{self.form}" + (
            f"{self.c_q2}x{self.c_k2}" if self.form == "repeat" else "")
        return (f"{self.name}:B{self.B}H{self.H}T{self.T}d{self.d}"
                f"_cq{self.c_q}ck{self.c_k}ch{self.c_h}_kq{kq}_head{hd}{form}_{self.dtype}")


def _configs() -> Dict[str, MTAConfig]:
    c = {}
    c["tiny"] = MTAConfig("tiny", B=1, H=4, T=128, d=32, c_q=3, c_k=5, c_h=2,
                          dtype="f32", qkv_std=1.0, theta_std=0.05, head_std=0.05,
                          layer=1, seed=1000)
    c["toy"] = MTAConfig("toy", B=64, H=4, T=256, d=64, c_q=2, c_k=9, c_h=2,
                         dtype="f32", qkv_std=1.0, theta_std=0.1, head_std=0.1,
                         layer=1, seed=1001)
    s = 1.0 / math.sqrt(2.0)
    c["layer2k"] = MTAConfig("layer2k", B=4, H=16, T=2048, d=128, c_q=6, c_k=11, c_h=2,
                             dtype="bf16", qkv_std=s, theta_std=0.02, head_std=0.02,
                             layer=4, seed=1002)
    c["needle4k"] = MTAConfig("needle4k", B=2, H=16, T=4096, d=128, c_q=6, c_k=11, c_h=2,
                              dtype="bf16", qkv_std=s, theta_std=0.02, head_std=0.02,
                              layer=4, needles=6, seed=1003)
    # the same layer with the sigmoid-gated GroupNorm (no depth scale)
    c["needle4k_gated"] = replace(c["needle4k"], name="needle4k_gated", layer=1, gated=True)
    # the same layer with Eq. 4's exact causal indicator instead of two-pass masks
    c["needle4k_exact"] = replace(c["needle4k"], name="needle4k_exact", kq_place=PRE_EXACT)
    # the both-pre-softmax 3D convolution, and the repeated convolution after the
    # softmax ("Putting Everything Together"), on the same layer
    c["needle4k_3d"] = replace(c["needle4k"], name="needle4k_3d", form="3d", head_place=PRE)
    c["needle4k_repeat"] = replace(c["needle4k"], name="needle4k_repeat", form="repeat", c_q2=6, c_k2=11)
    # the same layer with larger head groups: all sixteen heads in one group
    # (the pages' default c_h) and two groups of eight, both masking forms
    c["needle4k_ch8"] = replace(c["needle4k"], name="needle4k_ch8", c_h=8)
    c["needle4k_ch16"] = replace(c["needle4k"], name="needle4k_ch16", c_h=16)
    c["needle4k_ch16_post"] = replace(c["needle4k"], name="needle4k_ch16_post", c_h=16, kq_place=POST)
    for (cq, ck) in ((4, 9), (6, 11), (8, 15)):
        for ch in (2, 4):
            for kq in (PRE, POST):
                nm = f"sweep8k_{cq}x{ck}_ch{ch}_{'pre' if kq == PRE else 'post'}"
                c[nm] = MTAConfig(nm, B=1, H=32, T=8192, d=128, c_q=cq, c_k=ck, c_h=ch,
                                  kq_place=kq, head_place=POST, dtype="bf16",
                                  qkv_std=1.0, theta_std=0.05, head_std=0.05,
                                  layer=24, seed=1004)
    return c


CONFIGS: Dict[str, MTAConfig] = _configs()
SWEEP: List[str] = [k for k in CONFIGS if k.startswith("sweep8k_")]
HEADLINE = "needle4k"


def small(name: str = "small", **kw) -> MTAConfig:
    """A small ad-hoc configuration for tests (defaults: fp32, identity+noise)."""
    base = dict(B=1, H=2, T=64, d=32, c_q=3, c_k=5, c_h=2, dtype="f32",
                qkv_std=1.0, theta_std=0.1, head_std=0.1, layer=1, seed=7)
    base.update(kw)
    return MTAConfig(name, **base)


def generate(cfg: MTAConfig, device: str = "cpu") -> Dict[str, torch.Tensor]:
    """Draw the inputs of one configuration.

    Order of draws from ``torch.Generator().manual_seed(cfg.seed)``: Q, K, V,
    key-query kernel noise, head kernel noise, GroupNorm affine (only if
    ``gn_random``), per-head gate logits (only if ``gated``), then the needle
    positions and directions.  Q, K, V are drawn
    in fp32 and rounded to the run dtype (round to nearest even); kernels and
    GroupNorm parameters stay fp32.
    """
    g = torch.Generator(device="cpu").manual_seed(cfg.seed)
    shp = (cfg.B, cfg.H, cfg.T, cfg.d)
    q = torch.randn(shp, generator=g) * cfg.qkv_std
    k = torch.randn(shp, generator=g) * cfg.qkv_std
    v = torch.randn(shp, generator=g) * cfg.qkv_std

    theta = torch.randn((cfg.H, cfg.c_q, cfg.c_k), generator=g) * cfg.theta_std
    theta[:, 0, cfg.c_k // 2] += 1.0           # delta at (i'=0, j'=0)
    w = torch.randn((cfg.groups, cfg.c_h, cfg.c_h), generator=g) * cfg.head_std
    w += torch.eye(cfg.c_h).expand(cfg.groups, cfg.c_h, cfg.c_h)

    if cfg.gn_random:
        gn_w = 1.0 + 0.5 * torch.randn((cfg.H, cfg.d), generator=g)
        gn_b = 0.5 * torch.randn((cfg.H, cfg.d), generator=g)
    else:
        gn_w = torch.ones((cfg.H, cfg.d))
        gn_b = torch.zeros((cfg.H, cfg.d))

    gate = None
    if cfg.gated:
        # gate logits centred on sigma(g) = 1/2
        gate = cfg.gate_std * torch.randn((cfg.H,), generator=g)

    if cfg.needles:
        # Multi-needle retrieval stand-in: per batch row, `needles` key
        # positions (uniform without replacement, in random order) carry
        # needle_scale (3 in the workloads) times a per-head direction u, and
        # the last `needle_queries` queries carry u.
        nq = min(cfg.needle_queries, cfg.T)
        span = max(cfg.T - nq, cfg.needles)
        for b in range(cfg.B):
            pos = torch.randperm(span, generator=g)[: cfg.needles]
            for h in range(cfg.H):
                u = torch.randn((cfg.d,), generator=g) * cfg.qkv_std
                if cfg.needle_on_key:
                    k[b, h, pos] += cfg.needle_scale * u
                else:
                    k[b, h, pos] = cfg.needle_scale * u
                q[b, h, cfg.T - nq:] += u

    # kernels of the 3D and repeated forms, drawn after everything else so that
    # the other inputs do not depend on the form
    theta3 = theta2 = w2 = None
    if cfg.form == "3d":
        theta3 = torch.randn((cfg.groups, cfg.c_h, cfg.c_h, cfg.c_q, cfg.c_k), generator=g) * cfg.theta_std
        for a in range(cfg.c_h):
            theta3[:, a, a, 0, cfg.c_k // 2] += 1.0  # identity: each head's own delta
    elif cfg.form == "repeat":
        theta2 = torch.randn((cfg.H, cfg.c_q2, cfg.c_k2), generator=g) * cfg.theta_std
        theta2[:, 0, cfg.c_k2 // 2] += 1.0
        w2 = torch.randn((cfg.groups, cfg.c_h, cfg.c_h), generator=g) * cfg.head_std
        w2 += torch.eye(cfg.c_h).expand(cfg.groups, cfg.c_h, cfg.c_h)

    dt = DTYPES[cfg.dtype]
    out = {
        "q": q.to(dt).contiguous(),
        "k": k.to(dt).contiguous(),
        "v": v.to(dt).contiguous(),
        "theta_kq": theta.float().contiguous(),
        "theta_head": w.float().contiguous(),
        "gn_w": gn_w.float().contiguous(),
        "gn_b": gn_b.float().contiguous(),
    }
    if gate is not None:
        out["gate"] = gate.float().contiguous()
    if theta3 is not None:
        out["theta_3d"] = theta3.float().contiguous()
    if theta2 is not None:
        out["theta_kq2"] = theta2.float().contiguous()
        out["theta_head2"] = w2.float().contiguous()
    if device != "cpu":
        out = {kk: t.to(device) for kk, t in out.items()}
    return out


def layer_weights(cfg: MTAConfig, inp: Dict[str, torch.Tensor]) -> Dict:
    """The kernels of a configuration as stages of the general layer (kq_pre,
    head_pre, conv3d, head_post, kq_post, head_post2; absent stages omitted)
    plus the flags exact, c_q2, c_k2.  Pure bookkeeping of which tensor fills
    which stage."""
    exact = cfg.kq_place == PRE_EXACT
    if cfg.form == "3d":
        return {"conv3d": inp["theta_3d"], "exact": exact}
    if cfg.form == "repeat":
        return {"kq_pre": inp["theta_kq"], "head_post": inp["theta_head"], "kq_post": inp["theta_kq2"],
                "head_post2": inp["theta_head2"], "exact": exact, "c_q2": cfg.c_q2, "c_k2": cfg.c_k2}
    w = {"exact": exact}
    if cfg.kq_place == POST:
        w.update(kq_post=inp["theta_kq"], c_q2=cfg.c_q, c_k2=cfg.c_k)
    else:
        w["kq_pre"] = inp["theta_kq"]
    # on the same side of the softmax the key-query convolution comes first
    if cfg.head_place == PRE:
        w["head_pre"] = inp["theta_head"]
    else:
        w["head_post2" if cfg.kq_place == POST else "head_post"] = inp["theta_head"]
    return w


def with_(cfg: MTAConfig, **kw) -> MTAConfig:
    return replace(cfg, **kw)
