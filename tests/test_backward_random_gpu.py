"""Randomised backward parity: seeded draws of small configurations over both
backward forms (fused per tile, and the per-head maps in the workspace), every
placement of both convolutions, the exact indicator, c_h in {1, 2, 4}, both
dtypes, d in {32, 64, 128}, ragged and tiny T, gates and a random GroupNorm
affine; each gradient compared with the gradient oracle under the same bars
as tests/test_backward_gpu.py."""
import random

import numpy as np
import pytest
import torch

import test_backward_gpu as tb
from helpers import to_dev
from transformer_attention_variant_amd import binding
from transformer_attention_variant_amd import inputs as I

pytestmark = pytest.mark.gpu

SIZES = [(1, 1), (4, 9), (6, 11), (8, 15), (3, 5), (2, 4)]


def draw(i: int) -> I.MTAConfig:
    rng = random.Random(4242 + i)
    hs = rng.random() < 0.5  # half in the fused head-split scope (bf16, d = 128, compile-time sizes)
    dt = "bf16" if hs else rng.choice(["bf16", "f32"])
    d = 128 if hs else rng.choice([32, 64, 128])
    ch = rng.choice([1, 2, 2, 4])
    cq, ck = rng.choice(SIZES[:4] if hs else SIZES)
    return I.small(f"brnd{i}", B=rng.choice([1, 2]), H=ch * rng.choice([1, 2]),
                   T=rng.choice([1, 3, 17, 64, 65, 100, 130]), d=d, c_q=cq, c_k=ck, c_h=ch, dtype=dt,
                   kq_place=rng.choice([I.PRE, I.PRE, I.POST, I.PRE_EXACT]),
                   head_place=rng.choice([I.POST, I.POST, I.PRE]), qkv_std=0.7071 if dt == "bf16" else 1.0,
                   theta_std=rng.choice([0.02, 0.05, 0.1]), head_std=rng.choice([0.02, 0.05, 0.1]),
                   gated=rng.random() < 0.3, gn_random=rng.random() < 0.3, layer=rng.choice([1, 4]), seed=9500 + i)


@pytest.mark.parametrize("i", range(24))
def test_random_backward(i):
    cfg = draw(i)
    kname = binding.backward_kernel_name(cfg)
    if kname is None:
        pytest.skip(f"unsupported: {cfg.short()}")
    tb._say(f"[bwd random] {cfg.short()} gated={cfg.gated} -> {kname[:50]}")
    inp = I.generate(cfg)
    dout = tb._dout(cfg)
    got = binding.backward_cfg(cfg, to_dev(inp), dout.cuda())
    torch.cuda.synchronize()
    ref = tb._reference(cfg, inp, dout)
    scales = {n[len("scale_"):]: ref.pop(n).numpy() for n in list(ref) if n.startswith("scale_")}
    assert set(got) == set(ref)
    tol = tb.TOL["f32"] if kname.startswith("mta_bwd_gen") else tb.TOL[cfg.dtype]
    for name in ref:
        g = got[name].double().cpu().numpy()
        r = ref[name].numpy()
        assert np.isfinite(g).all(), name
        if name in scales:
            worst = float(np.max(np.abs(g - r) / np.maximum(tol * scales[name], 1e-300)))
            assert worst <= 1.0, f"{name}: error exceeds tol x term scale by {worst:.2f}x"
        else:
            rms = float(np.sqrt(np.mean(r ** 2)))
            rms_v = float(np.sqrt(np.mean(ref["v"].numpy() ** 2)))
            scale = rms if rms > 1e-9 * rms_v else rms_v
            err = float(np.max(np.abs(g - r)))
            assert err <= tol * scale, f"{name}: max abs err {err:.3e} > {tol * scale:.3e}"
