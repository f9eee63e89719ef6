"""GPU parity: the HIP path (called through the C ABI) against the CPU oracle on
the same seeded inputs.

* small shapes, compared element by element in full: every placement of the
  two convolutions, c_h in {1,2,4,8,16}, ragged T (tails of the 64-row tiles,
  T = 1, T < c_q), d in {32,64,128}, both dtypes, compile-time and runtime-
  sized stencils, even c_k, the largest kernel (16 x 31);
* the five workloads at their full sizes in the launch configuration the
  benchmark times: the two fp32 ones in full, the bf16 ones on sampled rows
  (sequence start, a tile boundary in the middle, the end) of sampled
  (batch, head group) units, which the oracle computes one by one;
* properties at full size: causality (perturbing the future leaves the past
  bitwise unchanged), determinism (two runs bitwise equal);
* empty inputs.
Tolerance, element by element: 1e-4 in fp32; in bf16 2e-2 x RMS(oracle output)
plus the bf16 unit roundoff 2^-8 x |oracle output| (the output's own rounding
to bf16), one rule for every bf16 case.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from helpers import compare, oracle_sampled, run_gpu, sample_plan, to_dev
from transformer_attention_variant_amd import binding
from transformer_attention_variant_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _small_cases():
    P, Q = I.PRE, I.POST
    c = []
    # fp32, fast stencils (3x5 @ d32, 2x9 @ d64) over placements / c_h / ragged T
    for kq in (P, Q):
        for hd in (Q, P):
            c.append(I.small(f"f32_d32_3x5_kq{kq}_h{hd}", B=2, H=4, T=100, d=32, c_q=3, c_k=5, c_h=2,
                             kq_place=kq, head_place=hd, seed=101 + 2 * kq + hd))
    for ch in (1, 2, 4):
        c.append(I.small(f"f32_d64_2x9_ch{ch}", B=1, H=4, T=130, d=64, c_q=2, c_k=9, c_h=ch, seed=110 + ch))
    # bf16 d128, the workload kernel sizes, ragged T, both kq placements
    for (cq, ck) in ((6, 11), (4, 9), (8, 15), (8, 13), (1, 1)):
        for kq in (P, Q):
            for ch in (2, 4):
                c.append(I.small(f"bf16_{cq}x{ck}_kq{kq}_ch{ch}", B=1, H=4, T=197, d=128, c_q=cq, c_k=ck,
                                 c_h=ch, kq_place=kq, dtype="bf16", qkv_std=0.7071, theta_std=0.05,
                                 head_std=0.05, seed=200 + cq * 10 + ck + kq + ch))
    # head mix before the softmax at c_h = 2 (the head-split kernel's 3D form with
    # the kernel w_ab theta_b): the instantiated sizes, ragged T, one tile + 1
    for (cq, ck, T) in ((6, 11, 197), (1, 1, 197), (6, 11, 65)):
        c.append(I.small(f"bf16_{cq}x{ck}_hpre_T{T}", B=2, H=4, T=T, d=128, c_q=cq, c_k=ck, c_h=2, kq_place=P,
                         head_place=P, dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.3,
                         seed=260 + cq + T))
    # one head per group: head pairs of single-head groups on the head-split
    # kernel (one pass before the softmax, two after it); odd H: the general kernel
    for kq in (P, I.PRE_EXACT, Q):
        c.append(I.small(f"bf16_6x11_ch1_kq{kq}", B=2, H=2, T=150, d=128, c_q=6, c_k=11, c_h=1, kq_place=kq,
                         dtype="bf16", qkv_std=0.7071, theta_std=0.05, seed=250 + kq))
    for (cq, ck, T) in ((4, 9, 197), (8, 15, 65), (1, 1, 130)):
        c.append(I.small(f"bf16_{cq}x{ck}_ch1_post_T{T}", B=1, H=4, T=T, d=128, c_q=cq, c_k=ck, c_h=1,
                         kq_place=Q, dtype="bf16", qkv_std=0.7071, theta_std=0.05, seed=255 + cq + T))
    c.append(I.small("bf16_6x11_ch1_post_H3", B=1, H=3, T=150, d=128, c_q=6, c_k=11, c_h=1, kq_place=Q,
                     dtype="bf16", qkv_std=0.7071, theta_std=0.05, seed=259))
    # one head per group with the 1x1 head mix before the softmax (it scales the
    # logits): the general kernel, every key-query placement, even and odd H
    for kq in (P, I.PRE_EXACT, Q):
        c.append(I.small(f"bf16_6x11_ch1_hpre_kq{kq}", B=2, H=2, T=128, d=128, c_q=6, c_k=11, c_h=1, kq_place=kq,
                         head_place=P, dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.3, gn_random=True,
                         seed=270 + kq))
    c.append(I.small("bf16_4x9_ch1_hpre_gated", B=3, H=4, T=65, d=128, c_q=4, c_k=9, c_h=1, kq_place=P,
                     head_place=P, dtype="bf16", qkv_std=0.7071, theta_std=0.1, head_std=0.3, gated=True,
                     gn_random=True, seed=274))
    c.append(I.small("f32_6x11_ch1_hpre_H3", B=1, H=3, T=100, d=64, c_q=6, c_k=11, c_h=1, kq_place=Q,
                     head_place=P, theta_std=0.05, head_std=0.3, seed=275))
    # runtime-sized stencils: odd/even c_k, head mix before the softmax, d in {32,64,128}
    for (d, dt) in ((32, "bf16"), (64, "bf16"), (128, "f32"), (128, "bf16")):
        for kq in (P, Q):
            for hd in (P, Q):
                c.append(I.small(f"gen_{dt}_d{d}_kq{kq}_h{hd}", B=2, H=4, T=77, d=d, c_q=5, c_k=4, c_h=2,
                                 kq_place=kq, head_place=hd, dtype=dt, seed=300 + d + 2 * kq + hd))
    # largest kernel, c_h = 1 and 4 with pre-softmax mixing
    c.append(I.small("gen_max_16x31", B=1, H=4, T=150, d=64, c_q=16, c_k=31, c_h=4, head_place=P, seed=401))
    c.append(I.small("gen_max_16x31_post", B=1, H=4, T=150, d=64, c_q=16, c_k=31, c_h=1,
                     kq_place=Q, seed=402))
    # sigmoid-gated GroupNorm, on both kernels and both dtypes
    for kq in (P, Q):
        c.append(I.small(f"gated_f32_kq{kq}", B=1, H=4, T=90, d=64, c_q=3, c_k=5, c_h=2, kq_place=kq,
                         gated=True, gate_std=3.0, gn_random=True, layer=3, seed=700 + kq))
        c.append(I.small(f"gated_bf16_kq{kq}", B=1, H=4, T=130, d=128, c_q=6, c_k=11, c_h=2, kq_place=kq,
                         dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.05, gated=True,
                         gate_std=1.0, gn_random=True, seed=710 + kq))
    # large competing logits: needle keys 9u on top of their own draw, so the
    # needles of a row reach ~50 natural units a few units apart (the sharpest
    # test of the convolution's operand precision before the softmax), both
    # masking forms, the instantiated sizes, one and several tiles
    for kq in (P, I.PRE_EXACT):
        for (cq, ck, T) in ((6, 11, 256), (8, 15, 200), (4, 9, 130), (1, 1, 256)):
            c.append(I.small(f"hot_bf16_{cq}x{ck}_kq{kq}_T{T}", B=1, H=4, T=T, d=128, c_q=cq, c_k=ck, c_h=2,
                             kq_place=kq, dtype="bf16", qkv_std=0.7071, theta_std=0.02, head_std=0.02,
                             layer=4, needles=6, needle_scale=9.0, needle_on_key=True,
                             seed=730 + cq + T + kq))
        # the same through single-head groups (head pairs; odd H: the general
        # kernel) and four-head groups
        for (ch, H, cq, ck) in ((1, 2, 6, 11), (1, 3, 6, 11), (4, 4, 6, 11), (4, 4, 8, 15), (16, 16, 6, 11)):
            c.append(I.small(f"hot_bf16_ch{ch}_H{H}_{cq}x{ck}_kq{kq}", B=1, H=H, T=256, d=128, c_q=cq, c_k=ck,
                             c_h=ch, kq_place=kq, dtype="bf16", qkv_std=0.7071, theta_std=0.02, head_std=0.02,
                             layer=4, needles=6, needle_scale=9.0, needle_on_key=True, seed=760 + ch + H + kq))
    # four-head groups on the head-split kernel (one workgroup per output head
    # pair, one sweep per source pair): two groups, every instantiated size and
    # placement, the workloads' near-identity mixing (weights N(0, 0.05) around
    # I: the pairs' cross terms carry a few percent of each output)
    for (cq, ck, kq) in ((6, 11, P), (6, 11, I.PRE_EXACT), (4, 9, Q), (8, 15, P), (8, 15, Q), (1, 1, Q)):
        c.append(I.small(f"quad_bf16_{cq}x{ck}_kq{kq}", B=2, H=8, T=150, d=128, c_q=cq, c_k=ck, c_h=4,
                         kq_place=kq, dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.05,
                         seed=900 + cq + ck + kq))
    for kq in (P, Q):
        c.append(I.small(f"quad_bf16_gated_kq{kq}", B=2, H=8, T=150, d=128, c_q=6, c_k=11, c_h=4, kq_place=kq,
                         dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.05, gated=True,
                         gate_std=1.0, gn_random=True, seed=940 + kq))
    # groups of 8 and 16 heads (c_h / 2 source-pair sweeps per output pair,
    # the probabilities in P.V as a bf16 high part and remainder): the
    # workloads' near-identity mix and dense ones (weights N(0, 0.5) around I:
    # every source head carries a large share of each output, and for some
    # output heads the weighted maps nearly cancel, so that one bf16 rounding
    # of each source head's probabilities before the mix would exceed the bar)
    for (ch, cq, ck, kq, hs) in ((8, 6, 11, P, 0.05), (8, 6, 11, I.PRE_EXACT, 0.05), (8, 4, 9, Q, 0.05),
                                 (8, 8, 15, P, 0.5), (8, 1, 1, Q, 0.5), (16, 6, 11, P, 0.05),
                                 (16, 6, 11, P, 0.5), (16, 8, 15, Q, 0.5), (16, 4, 9, I.PRE_EXACT, 0.5)):
        c.append(I.small(f"wide_bf16_ch{ch}_{cq}x{ck}_kq{kq}_w{hs}", B=1, H=16, T=150, d=128, c_q=cq, c_k=ck,
                         c_h=ch, kq_place=kq, dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=hs,
                         seed=970 + ch + cq + kq + int(hs * 10)))
    c.append(I.small("wide_bf16_ch16_gated", B=1, H=16, T=130, d=128, c_q=6, c_k=11, c_h=16, dtype="bf16",
                     qkv_std=0.7071, theta_std=0.05, head_std=0.05, gated=True, gate_std=1.0, gn_random=True,
                     seed=990))
    for T in (1, 65):
        for kq in (P, Q):
            c.append(I.small(f"wide_bf16_ch16_T{T}_kq{kq}", B=2, H=16, T=T, d=128, c_q=6, c_k=11, c_h=16,
                             kq_place=kq, dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.3,
                             seed=992 + T + kq))
    for T in (1, 3, 64, 65):
        for kq in (P, Q):
            c.append(I.small(f"quad_bf16_T{T}_kq{kq}", B=1, H=4, T=T, d=128, c_q=6, c_k=11, c_h=4, kq_place=kq,
                             dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.05, seed=950 + T + kq))
    # key-query convolution with Eq. 4's exact indicator: fast and runtime-sized
    # stencils, odd and even c_k, pre-softmax head mix, c_h = 4, both dtypes
    E = I.PRE_EXACT
    c.append(I.small("exact_f32_d32_3x5", B=2, H=4, T=100, d=32, c_q=3, c_k=5, c_h=2, kq_place=E,
                     theta_std=0.3, seed=801))
    c.append(I.small("exact_f32_d64_2x9_ch4", B=1, H=4, T=130, d=64, c_q=2, c_k=9, c_h=4, kq_place=E,
                     theta_std=0.3, seed=802))
    c.append(I.small("exact_f32_d64_5x4_hpre", B=1, H=4, T=77, d=64, c_q=5, c_k=4, c_h=2, kq_place=E,
                     head_place=P, theta_std=0.3, seed=803))
    c.append(I.small("exact_f32_16x31", B=1, H=2, T=150, d=64, c_q=16, c_k=31, c_h=1, kq_place=E,
                     seed=804))
    for (cq, ck) in ((6, 11), (4, 9), (8, 15), (1, 1)):
        c.append(I.small(f"exact_bf16_{cq}x{ck}", B=1, H=4, T=197, d=128, c_q=cq, c_k=ck, c_h=2,
                         kq_place=E, dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.05,
                         seed=810 + cq))
    # the pages' 8x13 ablation size (Table 5), with the exact indicator and single-head groups
    c.append(I.small("exact_bf16_8x13", B=1, H=4, T=197, d=128, c_q=8, c_k=13, c_h=2, kq_place=E,
                     dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.05, seed=830))
    c.append(I.small("bf16_8x13_ch1_post_T130", B=1, H=4, T=130, d=128, c_q=8, c_k=13, c_h=1, kq_place=Q,
                     dtype="bf16", qkv_std=0.7071, theta_std=0.05, seed=831))
    c.append(I.small("exact_bf16_5x4_d64", B=2, H=4, T=77, d=64, c_q=5, c_k=4, c_h=2, kq_place=E,
                     dtype="bf16", seed=820))
    c.append(I.small("exact_f32_T3", B=1, H=2, T=3, d=32, c_q=4, c_k=5, c_h=2, kq_place=E, seed=821))
    # tiny sequences: T = 1, T < c_q, exactly one tile, one tile + 1 (the
    # one-pass kernels' diagonal-only and ragged single/double tiles included)
    for T in (1, 3, 64, 65):
        c.append(I.small(f"f32_T{T}", B=2, H=2, T=T, d=32, c_q=3, c_k=5, c_h=2, seed=500 + T))
        c.append(I.small(f"bf16_T{T}_post", B=1, H=2, T=T, d=128, c_q=6, c_k=11, c_h=2, kq_place=Q,
                         dtype="bf16", seed=600 + T))
        for kq in (P, E):
            c.append(I.small(f"bf16_T{T}_kq{kq}", B=2, H=4, T=T, d=128, c_q=6, c_k=11, c_h=2, kq_place=kq,
                             dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.05, seed=650 + T + kq))
    return c


SMALL = _small_cases()


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_full(cfg):
    _say(f"[parity] small {cfg.short()}")
    inp = I.generate(cfg)
    got = run_gpu(cfg, inp)
    ref = oracle.forward_cfg(cfg, inp)
    err, tol = compare(cfg, got, ref, what="small")
    _say(f"[parity]   closest element: err {err:.3e} of bar {tol:.3e}")


@pytest.mark.parametrize("name", ["tiny", "toy"])
def test_workload_fp32_full(name):
    cfg = I.CONFIGS[name]
    _say(f"[parity] full {cfg.short()}")
    inp = I.generate(cfg)
    got = run_gpu(cfg, inp)
    ref = oracle.forward_cfg(cfg, inp)
    err, tol = compare(cfg, got, ref, what="full")
    _say(f"[parity]   max abs err {err:.3e} (tol {tol:.1e})")


@pytest.mark.parametrize("name", ["layer2k", "needle4k", "needle4k_gated", "needle4k_exact", "needle4k_ch8",
                                  "needle4k_ch16", "needle4k_ch16_post"] + I.SWEEP)
def test_workload_bf16_sampled(name):
    cfg = I.CONFIGS[name]
    _say(f"[parity] sampled {cfg.short()}")
    inp = I.generate(cfg)
    got = run_gpu(cfg, inp)
    ranges, units = sample_plan(cfg)
    ref, mask = oracle_sampled(cfg, inp, ranges, units)
    err, tol = compare(cfg, got, ref, mask=mask, what="sampled")
    assert np.isfinite(got.float().cpu().numpy()).all()
    _say(f"[parity]   rows {ranges} units {units}: max abs err {err:.3e} (tol {tol:.2e})")


@pytest.mark.parametrize("name", ["needle4k", "needle4k_exact", "sweep8k_8x15_ch4_post", "sweep8k_4x9_ch2_post"])
def test_causality_full_size(name):
    """Perturbing q, k, v after position t leaves out[..., :t+1, :] bitwise equal."""
    cfg = I.CONFIGS[name]
    _say(f"[parity] causality {cfg.short()}")
    inp = I.generate(cfg)
    dev = to_dev(inp)
    base = run_gpu(cfg, inp, dev).clone()
    t = cfg.T // 2 + 13
    g = torch.Generator(device="cpu").manual_seed(5)
    for name_ in ("q", "k", "v"):
        pert = dict(dev)
        x = pert[name_].clone()
        noise = torch.randn(x[:, :, t + 1:].shape, generator=g).to(x.dtype).cuda()
        x[:, :, t + 1:] += noise
        pert[name_] = x
        o2 = run_gpu(cfg, inp, pert)
        assert torch.equal(base[:, :, :t + 1], o2[:, :, :t + 1]), name_
        assert not torch.equal(base[:, :, t + 1:], o2[:, :, t + 1:]), name_


@pytest.mark.parametrize("name", ["needle4k", "toy"])
def test_determinism(name):
    cfg = I.CONFIGS[name]
    _say(f"[parity] determinism {cfg.short()}")
    inp = I.generate(cfg)
    dev = to_dev(inp)
    a = run_gpu(cfg, inp, dev).clone()
    b = run_gpu(cfg, inp, dev)
    assert torch.equal(a, b)


def test_identity_kernels_match_sdpa():
    """Identity kernels: the GPU output equals GroupNorm(causal SDPA) computed
    by torch on the CPU in float64 (a library routine, not the oracle)."""
    cfg = I.small("identity", B=2, H=4, T=150, d=64, c_q=4, c_k=7, c_h=2, dtype="f32", gn_random=True,
                  layer=5, seed=77)
    inp = I.generate(cfg)
    inp["theta_kq"].zero_()
    inp["theta_kq"][:, 0, cfg.c_k // 2] = 1.0
    inp["theta_head"] = torch.eye(2).expand(2, 2, 2).contiguous()
    got = run_gpu(cfg, inp).double().cpu()
    import torch.nn.functional as F
    o = F.scaled_dot_product_attention(inp["q"].double(), inp["k"].double(), inp["v"].double(),
                                       is_causal=True)
    x = o.permute(0, 2, 1, 3).reshape(cfg.B * cfg.T, cfg.H * cfg.d)
    y = F.group_norm(x, cfg.H, inp["gn_w"].double().reshape(-1), inp["gn_b"].double().reshape(-1),
                     cfg.gn_eps).reshape(cfg.B, cfg.T, cfg.H, cfg.d).permute(0, 2, 1, 3) * cfg.depth_scale
    assert float((got - y).abs().max()) <= 1e-4


def test_empty_inputs():
    for (B, T) in ((0, 16), (2, 0)):
        cfg = I.small("empty", B=B, H=2, T=T, d=32, c_h=2)
        dev = to_dev(I.generate(cfg))
        out = binding.forward_cfg(cfg, dev)
        torch.cuda.synchronize()
        assert out.numel() == 0


def test_out_argument_and_stream():
    cfg = I.small("outarg", B=1, H=2, T=70, d=32, c_q=3, c_k=5, c_h=2, seed=9)
    inp = I.generate(cfg)
    dev = to_dev(inp)
    s = torch.cuda.Stream()
    out = torch.full_like(dev["q"], float("nan"))
    with torch.cuda.stream(s):
        binding.forward_cfg(cfg, dev, out=out, stream=s)
    s.synchronize()
    compare(cfg, out, oracle.forward_cfg(cfg, inp), what="out/stream")
