"""The allocation-free backward entry point (mta_backward_noalloc, whose
workspace is the library's device scratch array) against mta_backward with a
caller workspace, through the C ABI: two calls in a row on one GPU, the second
with a smaller problem (the scratch array keeps the first call's contents), and
the host-side refusal of a problem larger than the array."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from helpers import to_dev
from transformer_attention_variant_amd import binding
from transformer_attention_variant_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dout(cfg):
    g = torch.Generator().manual_seed(cfg.seed + 17)
    return torch.randn((cfg.B, cfg.H, cfg.T, cfg.d), generator=g).to(I.DTYPES[cfg.dtype])


def _check_same(cfg, a, b):
    """dk, dv bitwise (no atomics); the rest (sums with atomics in arbitrary
    order) to rounding."""
    assert set(a) == set(b)
    assert torch.equal(a["k"], b["k"]) and torch.equal(a["v"], b["v"])
    for n in a:
        x, y = a[n].double().cpu().numpy(), b[n].double().cpu().numpy()
        assert np.isfinite(x).all() and np.isfinite(y).all(), n
        scale = float(np.max(np.abs(y))) or 1.0
        err = float(np.max(np.abs(x - y)))
        _say(f"[noalloc]   {n:10s} max abs diff {err:.3e} (scale {scale:.3e})")
        assert err <= 1e-5 * scale, f"{n}: {err:.3e} vs scale {scale:.3e}"


def test_noalloc_matches_workspace_entry_point():
    lib = binding.load()
    cases = [I.small("noalloc_big", B=2, H=4, T=300, d=128, c_q=6, c_k=11, c_h=2, dtype="bf16", qkv_std=0.7071,
                     theta_std=0.05, head_std=0.05, gated=True, gn_random=True, seed=1501),
             I.small("noalloc_small", B=1, H=2, T=97, d=128, c_q=4, c_k=9, c_h=2, kq_place=I.PRE_EXACT,
                     dtype="bf16", qkv_std=0.7071, theta_std=0.05, head_std=0.05, seed=1502),
             # the backward that keeps its maps in the workspace (convolution after the softmax, c_h = 4)
             I.small("noalloc_maps", B=1, H=4, T=130, d=64, c_q=4, c_k=9, c_h=4, kq_place=I.POST, dtype="bf16",
                     theta_std=0.1, head_std=0.1, gn_random=True, seed=1503)]
    for cfg in cases:
        _say(f"[noalloc] {cfg.short()}")
        c = binding.make_config(cfg.B, cfg.H, cfg.T, cfg.d, cfg.c_q, cfg.c_k, cfg.c_h, cfg.kq_place,
                                cfg.head_place, I.BF16, cfg.gn_eps, cfg.depth_scale)
        assert lib.mta_backward_workspace_size(ctypes.byref(c)) <= lib.mta_backward_scratch_bytes()
        inp = I.generate(cfg)
        dev = to_dev(inp)
        dout = _dout(cfg).cuda()
        got = binding.backward_cfg(cfg, dev, dout, noalloc=True)
        ref = binding.backward_cfg(cfg, dev, dout)
        torch.cuda.synchronize()
        _check_same(cfg, got, ref)


@pytest.mark.parametrize("name", ["sweep8k_6x11_ch2_pre", "sweep8k_6x11_ch4_post"])
def test_noalloc_refuses_problems_beyond_its_scratch(name):
    lib = binding.load()
    cfg = I.CONFIGS[name]
    c = binding.make_config(cfg.B, cfg.H, cfg.T, cfg.d, cfg.c_q, cfg.c_k, cfg.c_h, cfg.kq_place, cfg.head_place,
                            I.BF16, cfg.gn_eps, cfg.depth_scale)
    assert lib.mta_backward_workspace_size(ctypes.byref(c)) > lib.mta_backward_scratch_bytes()
    good = 0x10000  # never dereferenced: the call returns during validation
    rc = lib.mta_backward_noalloc(*([good] * 9), ctypes.byref(c), *([good] * 9), None)
    assert rc == -9 and binding.status_string(rc)
