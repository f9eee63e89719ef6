"""The C-ABI library: it loads, exports every symbol include/mta.h declares,
and its host-side validation returns the documented codes before any device
work (these tests make no GPU call and run without a GPU)."""
import ctypes
import os
import re

import pytest

from transformer_attention_variant_amd import binding
from transformer_attention_variant_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from transformer_attention_variant_amd import build
        build.build()
    return binding.load()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mta.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mta_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


@pytest.mark.parametrize("name,expect", [
    ("needle4k", "mta_fwd_v4"), ("needle4k_exact", "mta_fwd_v4"), ("layer2k", "mta_fwd_v4"),
    ("sweep8k_8x15_ch2_pre", "mta_fwd_v4"),
    ("sweep8k_6x11_ch2_post", "mta_fwd_v4 (two passes"), ("sweep8k_4x9_ch2_post", "mta_fwd_v4 (two passes"),
    # c_h = 4: the head-split kernel per output head pair, one sweep per source pair
    ("sweep8k_8x15_ch4_pre", "mta_fwd_v4 (four-head groups: two source-pair sweeps, head-split"),
    ("sweep8k_6x11_ch4_post", "mta_fwd_v4 (four-head groups: two source-pair sweeps of two passes"),
    ("sweep8k_8x15_ch4_post", "mta_fwd_v4 (four-head groups: two source-pair sweeps of two passes"),
    ("toy", "mta_fwd_kernel"), ("tiny", "mta_fwd_kernel"),
    ("needle4k_ch8", "mta_fwd_v4 (groups of 8 or 16 heads: one source-pair sweep per head pair"),
    ("needle4k_ch16", "mta_fwd_v4 (groups of 8 or 16 heads: one source-pair sweep per head pair"),
    ("needle4k_ch16_post", "mta_fwd_v4 (groups of 8 or 16 heads: one source-pair sweep of two passes"),
    ("needle4k_3d", "mta_fwd_v4 (one pass, head-split waves, 3D"), ("needle4k_repeat", "mta_fwd_rep (two passes"),
])
def test_kernel_selection(lib, name, expect):
    """Host-only query of the kernel each workload runs (no launch)."""
    got = binding.kernel_name(I.CONFIGS[name])
    assert got is not None and got.startswith(expect), got


@pytest.mark.parametrize("kq,expect", [(I.PRE, "mta_fwd_v4 (one pass, head-split waves, pre-softmax head mix"),
                                       (I.PRE_EXACT, "mta_fwd_kernel"), (I.POST, "mta_fwd_kernel")])
def test_kernel_selection_head_mix_before_softmax(lib, kq, expect):
    """c_h = 2 with the head mix before the softmax: the head-split kernel's 3D form
    for the two-pass masks at an instantiated size, else the general kernel."""
    cfg = I.small("hpre", B=1, H=4, T=256, d=128, c_q=6, c_k=11, c_h=2, kq_place=kq, head_place=I.PRE,
                  dtype="bf16")
    got = binding.kernel_name(cfg)
    assert got is not None and got.startswith(expect), got


@pytest.mark.parametrize("kq,form", [(I.PRE, "one pass"), (I.PRE_EXACT, "one pass"), (I.POST, "two passes")])
def test_kernel_selection_single_head_groups(lib, kq, form):
    """Groups of one head run the head-split kernel two groups at a time when
    the head count is even, else the general kernel."""
    cfg = I.small("ch1", B=1, H=4, T=256, d=128, c_q=6, c_k=11, c_h=1, kq_place=kq, dtype="bf16")
    got = binding.kernel_name(cfg)
    assert got is not None and got.startswith(f"mta_fwd_v4 ({form}, head-split waves, head pairs"), got
    odd = I.with_(cfg, H=3)
    got = binding.kernel_name(odd)
    assert got is not None and got.startswith("mta_fwd_kernel"), got
    # the 1x1 head mix before the softmax scales the logits, which the head-pair
    # form does not do: the general kernel
    pre = I.with_(cfg, head_place=I.PRE)
    got = binding.kernel_name(pre)
    assert got is not None and got.startswith("mta_fwd_kernel"), got


def test_kernel_name_of_invalid_config(lib):
    assert lib.mta_kernel_name(None) is None
    c = cfg(c_h=3, H=6)
    assert lib.mta_kernel_name(ctypes.byref(c)) is None


def _layer(**kw):
    c = dict(B=2, H=4, T=100, d=128, c_q=6, c_k=11, c_q2=3, c_k2=5, c_h=2, exact=0, dtype=1, gn_eps=1e-5,
             depth_scale=1.0)
    c.update({k: v for k, v in kw.items() if k in c})
    cfg = binding.MtaLayerConfig(c["B"], c["H"], c["T"], c["d"], c["c_q"], c["c_k"], c["c_q2"], c["c_k2"],
                                 c["c_h"], c["exact"], c["dtype"], c["gn_eps"], c["depth_scale"])
    ptrs = dict(kq_pre=0x1000, head_post=0x1000, kq_post=0x1000, head_post2=0x1000, gn_w=0x1000, gn_b=0x1000)
    ptrs.update({k: v for k, v in kw.items() if k in binding.LAYER_KERNELS or k in ("gn_w", "gn_b", "gate")})
    w = binding.MtaLayerWeights(*[ptrs.get(n) for n in binding.LAYER_KERNELS], ptrs.get("gn_w"),
                                ptrs.get("gn_b"), ptrs.get("gate"))
    return cfg, w


@pytest.mark.parametrize("kw,code", [
    ({}, 0), (dict(B=0), 0),
    (dict(H=6, c_h=4), -2), (dict(c_q=0), -2), (dict(c_k2=0), -2),
    (dict(conv3d=0x1000), -3), (dict(exact=2), -3),
    (dict(dtype=3), -4), (dict(gn_eps=-1.0), -8),
    (dict(d=96), -6), (dict(c_q2=17), -6), (dict(c_k=32), -6),
    (dict(kq_post=None, c_q2=0), 0), (dict(kq_pre=None, c_q=0), 0),
])
def test_layer_validation(lib, kw, code):
    """mta_forward_layer validates on the host before any device work (the
    tensor pointers here are never dereferenced; B = 0 returns before them)."""
    cfg, w = _layer(**kw)
    if code == 0:
        got = lib.mta_layer_kernel_name(ctypes.byref(cfg), ctypes.byref(w))
        assert got is not None
    else:
        assert lib.mta_forward_layer(0x10000, 0x10000, 0x10000, ctypes.byref(w), ctypes.byref(cfg), 0x10000,
                                     None) == code
        assert lib.mta_layer_kernel_name(ctypes.byref(cfg), ctypes.byref(w)) is None
    assert lib.mta_forward_layer(None, None, None, None, ctypes.byref(cfg), None, None) == -1


@pytest.mark.parametrize("kw,expect", [
    ({}, "mta_fwd_layer"),                                                  # the repeated form, 6x11 then 3x5
    (dict(c_q2=6, c_k2=11), "mta_fwd_rep (two passes"),                     # 6x11 before and after: head-split
    (dict(c_q=4, c_k=9, c_q2=4, c_k2=9), "mta_fwd_rep (two passes"),
    (dict(c_q=1, c_k=1, c_q2=1, c_k2=1), "mta_fwd_rep (two passes"),
    (dict(c_q=6, c_k=11, c_q2=4, c_k2=9), "mta_fwd_layer"),                 # unequal sizes: general kernel
    (dict(c_q2=6, c_k2=11, head_post=None, head_post2=None), "mta_fwd_rep (two passes"),
    (dict(c_q2=6, c_k2=11, exact=1), "mta_fwd_layer"),                      # Eq. 4's indicator: general kernel
    (dict(c_q2=6, c_k2=11, dtype=0), "mta_fwd_layer"),                      # float32
    (dict(c_q2=6, c_k2=11, d=64), "mta_fwd_layer"),
    (dict(c_q2=6, c_k2=11, head_pre=0x1000), "mta_fwd_layer"),              # a head mix before the softmax
    (dict(kq_post=None, head_post2=None), "mta_fwd_v4"),                    # kq pre + head post
    (dict(kq_pre=None, head_post=None, c_q2=6, c_k2=11), "mta_fwd_v4 (two passes"),  # kq post + head post
    (dict(kq_pre=None, head_post2=None), "mta_fwd_layer"),                  # head mix before the kq conv
    (dict(kq_pre=None, head_post=None, head_post2=None, kq_post=None, conv3d=0x1000), "mta_fwd_v4 (one pass, head-split waves, 3D"),
    (dict(kq_pre=None, head_post=None, head_post2=None, kq_post=None, conv3d=0x1000, exact=1), "mta_fwd_layer"),
    (dict(kq_pre=None, head_post=None, head_post2=None, kq_post=None, conv3d=0x1000, c_q=3, c_k=5), "mta_fwd_layer"),
    (dict(kq_pre=None, kq_post=None, head_post2=None, conv3d=0x1000), "mta_fwd_layer"),   # 3D then a head mix
])
def test_layer_kernel_selection(lib, kw, expect):
    cfg, w = _layer(**kw)
    got = lib.mta_layer_kernel_name(ctypes.byref(cfg), ctypes.byref(w))
    assert got is not None and got.decode().startswith(expect), got


def test_backward_validation(lib):
    """mta_backward's host checks (no device work on these paths)."""
    good = 0x10000
    c = cfg()
    n = lib.mta_backward_workspace_size(ctypes.byref(c))
    assert n >= 2 * 4 * 100 * 128 * 2  # dO in bf16 at least
    args = lambda **kw: dict(dict(q=good, k=good, v=good, th=good, w=good, gw=good, gb=good, gate=None,
                                  dout=good, dq=good, dk=good, dv=good, dth=good, dw=good, dgw=good, dgb=good,
                                  dgate=None, ws=good, nws=n), **kw)

    def call(c_, **kw):
        a_ = args(**kw)
        return lib.mta_backward(a_["q"], a_["k"], a_["v"], a_["th"], a_["w"], a_["gw"], a_["gb"], a_["gate"],
                                a_["dout"], ctypes.byref(c_), a_["dq"], a_["dk"], a_["dv"], a_["dth"], a_["dw"],
                                a_["dgw"], a_["dgb"], a_["dgate"], a_["ws"], a_["nws"], None)
    # every other placement runs the backward with its maps in the workspace:
    # a workspace below one head group's maps is refused, so is T > 32768
    for other in (cfg(kq_place=1), cfg(head_place=0), cfg(H=8, c_h=4), cfg(H=8, c_h=8), cfg(H=16, c_h=16),
                  cfg(H=8, c_h=8, dtype=0, d=32)):
        name = lib.mta_backward_kernel_name(ctypes.byref(other))
        assert name is not None and name.decode().startswith("mta_bwd_gen"), name
        assert lib.mta_backward_workspace_size(ctypes.byref(other)) > 4096
        assert call(other, nws=4096) == -8
        assert call(cfg(kq_place=other.kq_place, head_place=other.head_place, H=other.heads, c_h=other.c_h,
                        T=40000)) == -6
    assert lib.mta_backward_kernel_name(ctypes.byref(c)).decode().startswith("mta_bwd (fused")
    assert call(c, dq=None) == -1
    assert call(c, gate=good, dgate=None) == -1
    assert call(c, ws=good + 16) == -5          # workspace not 256-byte aligned
    assert call(c, nws=n - 1) == -8             # workspace too small
    assert call(cfg(B=0)) == 0
    assert lib.mta_backward_workspace_size(None) == 0


def test_version_and_status_strings(lib):
    assert lib.mta_abi_version() == 100
    for code in list(binding.STATUS) + [-99]:
        s = lib.mta_status_string(code)
        assert s and len(s.decode()) > 0


def cfg(**kw):
    base = dict(B=2, H=4, T=100, d=128, c_q=6, c_k=11, c_h=2, kq_place=0, head_place=1, dtype=1,
                gn_eps=1e-5, depth_scale=0.5)
    base.update(kw)
    return binding.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    (dict(B=0), 0), (dict(T=0), 0),
    (dict(B=-1), -2), (dict(T=-5), -2), (dict(H=0), -2), (dict(d=0), -2),
    (dict(c_q=0), -2), (dict(c_k=0), -2), (dict(c_h=0), -2), (dict(H=6, c_h=4), -2),
    (dict(kq_place=2), 0), (dict(kq_place=3), -3), (dict(kq_place=-1), -3),
    (dict(head_place=-1), -3), (dict(head_place=2), -3),
    (dict(dtype=7), -4),
    (dict(gn_eps=0.0), -8), (dict(gn_eps=float("nan")), -8), (dict(depth_scale=float("inf")), -8),
    (dict(d=96), -6), (dict(d=256), -6), (dict(H=3, c_h=3), -6), (dict(H=12, c_h=6), -6),
    (dict(H=32, c_h=32), -6),
    # groups of 8 or 16 heads: the head-split kernel's source-pair sweeps only
    # (bf16, d = 128, head mix after the softmax, its compile-time kernel sizes)
    (dict(H=8, c_h=8), 0), (dict(H=16, c_h=16), 0), (dict(H=16, c_h=16, kq_place=1), 0),
    (dict(H=16, c_h=8, kq_place=2), 0), (dict(H=16, c_h=16, c_q=1, c_k=1), 0),
    (dict(H=8, c_h=8, dtype=0), -6), (dict(H=8, c_h=8, head_place=0), -6),
    (dict(H=8, c_h=8, c_q=5, c_k=7), -6), (dict(H=8, c_h=8, d=64), -6),
    (dict(c_q=17), -6), (dict(c_k=32), -6), (dict(T=(1 << 24) + 1), -6),
    (dict(c_q=16, c_k=31), 0), (dict(c_k=4), 0), (dict(d=32, dtype=0), 0),
])
def test_check_config(lib, kw, code):
    c = cfg(**kw)
    assert lib.mta_check_config(ctypes.byref(c)) == code


def test_check_config_includes_the_lds_fit(lib):
    # valid shape, but its kernel's LDS (fp32, d = 128, c_h = 4, 16x31, key-query
    # convolution after the softmax with the head mix before it) exceeds 160 KB:
    # mta_check_config returns what mta_forward would, and no kernel is named
    c = cfg(d=128, dtype=0, c_h=4, c_q=16, c_k=31, kq_place=1, head_place=0)
    assert lib.mta_check_config(ctypes.byref(c)) == -6
    assert lib.mta_kernel_name(ctypes.byref(c)) is None
    good = 0x10000  # never dereferenced: the call returns during planning
    assert lib.mta_forward(*([good] * 7), ctypes.byref(c), good, None) == -6


def test_forward_rejects_before_any_device_work(lib):
    c = cfg()
    good = 0x10000  # never dereferenced: every call below returns during validation
    args = [good] * 7
    assert lib.mta_forward(*args, None, good, None) == -1                 # NULL cfg
    bad = cfg(c_h=3)
    assert lib.mta_forward(*args, ctypes.byref(bad), good, None) == -2
    for i in range(7):
        a = list(args)
        a[i] = None
        assert lib.mta_forward(*a, ctypes.byref(c), good, None) == -1
    assert lib.mta_forward(*args, ctypes.byref(c), None, None) == -1      # NULL out
    for i in range(3):
        a = list(args)
        a[i] = good + 8                                                   # q/k/v not 16-byte aligned
        assert lib.mta_forward(*a, ctypes.byref(c), good, None) == -5
    assert lib.mta_forward(*args, ctypes.byref(c), good + 4, None) == -5  # out misaligned
    a = list(args)
    a[3] = good + 2                                                       # theta not 4-byte aligned
    assert lib.mta_forward(*a, ctypes.byref(c), good, None) == -5


def test_gated_entry_requires_gate(lib):
    c = cfg()
    good = 0x10000
    args = [good] * 7
    assert lib.mta_forward_gated(*args, None, ctypes.byref(c), good, None) == -1
    assert lib.mta_forward_gated(*args, good + 2, ctypes.byref(c), good, None) == -5
    bad = cfg(kq_place=5)
    assert lib.mta_forward_gated(*args, good, ctypes.byref(bad), good, None) == -3
    e = cfg(B=0)
    assert lib.mta_forward_gated(*([None] * 8), ctypes.byref(e), None, None) == 0


def test_empty_problem_launches_nothing(lib):
    # B == 0 or T == 0 succeeds without touching pointers (NULL is fine)
    for kw in (dict(B=0), dict(T=0)):
        c = cfg(**kw)
        assert lib.mta_forward(None, None, None, None, None, None, None, ctypes.byref(c), None, None) == 0


def test_config_layout_matches_header():
    # 10 int32 + 2 float32, no padding
    assert ctypes.sizeof(binding.MtaConfig) == 48
    names = [f[0] for f in binding.MtaConfig._fields_]
    src = open(os.path.join(ROOT, "include", "mta.h")).read()
    body = src[src.index("typedef struct mta_config"):src.index("} mta_config;")]
    hdr = re.findall(r"(?:int32_t|float)\s+(\w+);", body)
    assert hdr == names


def test_python_binding_refuses_cpu_tensors(lib):
    c = I.small(T=8)
    inp = I.generate(c)
    with pytest.raises(ValueError):
        binding.forward_cfg(c, inp)


@pytest.mark.parametrize("kq,ch,expect", [
    (I.PRE, 2, "mta_fwd_v4 (one pass"), (I.PRE_EXACT, 2, "mta_fwd_v4 (one pass"),
    (I.POST, 2, "mta_fwd_v4 (two passes"), (I.POST, 1, "mta_fwd_v4 (two passes, head-split waves, head pairs"),
    (I.PRE, 4, "mta_fwd_v4 (four-head groups"), (I.POST, 16, "mta_fwd_v4 (groups of 8 or 16 heads")])
def test_kernel_selection_8x13(lib, kq, ch, expect):
    """The 8x13 kernel of the pages' kernel-size ablation runs the head-split
    kernel in every family that the workload sizes run."""
    cfg = I.small("k8x13", B=1, H=16, T=256, d=128, c_q=8, c_k=13, c_h=ch, kq_place=kq, dtype="bf16")
    got = binding.kernel_name(cfg)
    assert got is not None and got.startswith(expect), got
