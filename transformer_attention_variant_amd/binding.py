"""Thin ctypes binding of the C ABI in include/mta.h.

Argument marshalling only: every step of the forward runs in the HIP kernels
of ``libmta.so``.  PyTorch supplies device memory and the stream.  There is no
fallback: without the built library, or without a GPU, ``forward`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

from . import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmta.so")

MTA_OK = 0
STATUS = {0: "MTA_OK", -1: "MTA_ERR_NULL_ARG", -2: "MTA_ERR_BAD_SHAPE", -3: "MTA_ERR_BAD_PLACEMENT",
          -4: "MTA_ERR_BAD_DTYPE", -5: "MTA_ERR_MISALIGNED", -6: "MTA_ERR_UNSUPPORTED",
          -7: "MTA_ERR_LAUNCH", -8: "MTA_ERR_BAD_VALUE", -9: "MTA_ERR_SCRATCH"}
# names declared in include/mta.h
EXPORTS = ("mta_forward", "mta_forward_gated", "mta_forward_layer", "mta_backward", "mta_backward_workspace_size",
           "mta_backward_noalloc", "mta_backward_scratch_bytes", "mta_backward_kernel_name", "mta_check_config",
           "mta_kernel_name", "mta_layer_kernel_name", "mta_status_string", "mta_abi_version")
LAYER_KERNELS = ("kq_pre", "head_pre", "conv3d", "head_post", "kq_post", "head_post2")


class MtaConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("c_q", ctypes.c_int32), ("c_k", ctypes.c_int32),
                ("c_h", ctypes.c_int32), ("kq_place", ctypes.c_int32), ("head_place", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("gn_eps", ctypes.c_float), ("depth_scale", ctypes.c_float)]


class MTAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class MtaLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_KERNELS] + \
        [("gn_w", ctypes.c_void_p), ("gn_b", ctypes.c_void_p), ("gate", ctypes.c_void_p)]


class MtaLayerConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("c_q", ctypes.c_int32), ("c_k", ctypes.c_int32),
                ("c_q2", ctypes.c_int32), ("c_k2", ctypes.c_int32), ("c_h", ctypes.c_int32),
                ("exact", ctypes.c_int32), ("dtype", ctypes.c_int32), ("gn_eps", ctypes.c_float),
                ("depth_scale", ctypes.c_float)]


_lib = None


def load(path: Optional[str] = None):
    """Load libmta.so (raises if it has not been built)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run transformer_attention_variant_amd/build.py "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    vp = ctypes.c_void_p
    lib.mta_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(MtaConfig), vp, vp]
    lib.mta_forward.restype = ctypes.c_int
    lib.mta_forward_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(MtaConfig), vp, vp]
    lib.mta_forward_gated.restype = ctypes.c_int
    lib.mta_check_config.argtypes = [ctypes.POINTER(MtaConfig)]
    lib.mta_check_config.restype = ctypes.c_int
    lib.mta_status_string.argtypes = [ctypes.c_int]
    lib.mta_status_string.restype = ctypes.c_char_p
    lib.mta_forward_layer.argtypes = [vp, vp, vp, ctypes.POINTER(MtaLayerWeights),
                                      ctypes.POINTER(MtaLayerConfig), vp, vp]
    lib.mta_forward_layer.restype = ctypes.c_int
    lib.mta_layer_kernel_name.argtypes = [ctypes.POINTER(MtaLayerConfig), ctypes.POINTER(MtaLayerWeights)]
    lib.mta_layer_kernel_name.restype = ctypes.c_char_p
    lib.mta_backward.argtypes = [vp] * 9 + [ctypes.POINTER(MtaConfig)] + [vp] * 9 + [ctypes.c_size_t, vp]
    lib.mta_backward.restype = ctypes.c_int
    lib.mta_backward_workspace_size.argtypes = [ctypes.POINTER(MtaConfig)]
    lib.mta_backward_workspace_size.restype = ctypes.c_size_t
    lib.mta_backward_noalloc.argtypes = [vp] * 9 + [ctypes.POINTER(MtaConfig)] + [vp] * 9
    lib.mta_backward_noalloc.restype = ctypes.c_int
    lib.mta_backward_scratch_bytes.argtypes = []
    lib.mta_backward_scratch_bytes.restype = ctypes.c_size_t
    lib.mta_kernel_name.argtypes = [ctypes.POINTER(MtaConfig)]
    lib.mta_kernel_name.restype = ctypes.c_char_p
    lib.mta_backward_kernel_name.argtypes = [ctypes.POINTER(MtaConfig)]
    lib.mta_backward_kernel_name.restype = ctypes.c_char_p
    lib.mta_abi_version.argtypes = []
    lib.mta_abi_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def make_config(B, H, T, d, c_q, c_k, c_h, kq_place=I.PRE, head_place=I.POST, dtype=I.BF16,
                gn_eps=1e-5, depth_scale=1.0) -> MtaConfig:
    return MtaConfig(B, H, T, d, c_q, c_k, c_h, kq_place, head_place, dtype, gn_eps, depth_scale)


def _layer_structs(B, H, T, d, dtype, c_h, c_q, c_k, c_q2, c_k2, exact, gn_eps, depth_scale, ptrs):
    cfg = MtaLayerConfig(B, H, T, d, c_q, c_k, c_q2, c_k2, c_h, int(bool(exact)), dtype, gn_eps, depth_scale)
    w = MtaLayerWeights(*[ptrs.get(n) for n in LAYER_KERNELS], ptrs.get("gn_w"), ptrs.get("gn_b"),
                        ptrs.get("gate"))
    return cfg, w


def kernel_name(cfg: I.MTAConfig) -> Optional[str]:
    """Name of the kernel the library launches for a workload configuration."""
    if cfg.form != "std":
        kinds = {n: 1 for n in LAYER_KERNELS if n in I.layer_weights(cfg, _shape_only(cfg))}
        kinds.update(gn_w=1, gn_b=1)
        lc, lw = _layer_structs(cfg.B, cfg.H, cfg.T, cfg.d, I.F32 if cfg.dtype == "f32" else I.BF16, cfg.c_h,
                                cfg.c_q, cfg.c_k, cfg.c_q2, cfg.c_k2, cfg.kq_place == I.PRE_EXACT, cfg.gn_eps,
                                cfg.depth_scale, kinds)
        r = load().mta_layer_kernel_name(ctypes.byref(lc), ctypes.byref(lw))
        return r.decode() if r else None
    c = make_config(cfg.B, cfg.H, cfg.T, cfg.d, cfg.c_q, cfg.c_k, cfg.c_h, cfg.kq_place, cfg.head_place,
                    I.F32 if cfg.dtype == "f32" else I.BF16, cfg.gn_eps, cfg.depth_scale)
    r = load().mta_kernel_name(ctypes.byref(c))
    return r.decode() if r else None


def _shape_only(cfg: I.MTAConfig) -> Dict:
    """Placeholders with the keys generate() would produce for `cfg` (no data)."""
    keys = ["q", "k", "v", "theta_kq", "theta_head", "gn_w", "gn_b"]
    keys += {"3d": ["theta_3d"], "repeat": ["theta_kq2", "theta_head2"]}.get(cfg.form, [])
    return {k: None for k in keys}


def _launch_stream(device, stream: Optional[torch.cuda.Stream]) -> torch.cuda.Stream:
    """The stream a call launches on: ``stream``, or torch's current stream.  A
    side stream first waits for the work already queued on the current stream
    (the inputs may still be in flight there)."""
    cur = torch.cuda.current_stream(device)
    if stream is None or stream.cuda_stream == cur.cuda_stream:
        return cur
    stream.wait_stream(cur)
    return stream


def status_string(code: int) -> str:
    return load().mta_status_string(int(code)).decode()


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, theta_kq: torch.Tensor,
            theta_head: torch.Tensor, gn_w: torch.Tensor, gn_b: torch.Tensor, *, c_q: int, c_k: int,
            c_h: int, kq_place: int = I.PRE, head_place: int = I.POST, gn_eps: float = 1e-5,
            depth_scale: float = 1.0, gate: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None,
            stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """MTA forward on the GPU through ``mta_forward`` (``mta_forward_gated``
    when a per-head ``gate`` [H] float32 tensor is given).  q, k, v: [B,H,T,d]
    float32 or bfloat16 CUDA tensors; theta_kq [H,c_q,c_k], theta_head
    [H/c_h,c_h,c_h], gn_w/gn_b [H,d] float32.  Asynchronous on ``stream``
    (default: torch's current stream)."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, H, T, d = q.shape
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q, k, v must be float32 or bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    for name, t in (("theta_kq", theta_kq), ("theta_head", theta_head), ("gn_w", gn_w), ("gn_b", gn_b)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("theta_kq", theta_kq), ("theta_head", theta_head),
                    ("gn_w", gn_w), ("gn_b", gn_b)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if gate is not None:
        if gate.dtype != torch.float32 or not gate.is_cuda or not gate.is_contiguous() \
                or tuple(gate.shape) != (H,):
            raise ValueError("gate must be a contiguous float32 CUDA tensor of shape [H]")
    if tuple(theta_kq.shape) != (H, c_q, c_k) or tuple(theta_head.shape) != (H // max(c_h, 1), c_h, c_h) \
            or tuple(gn_w.shape) != (H, d) or tuple(gn_b.shape) != (H, d):
        raise ValueError("parameter shapes do not match (theta_kq [H,c_q,c_k], theta_head [H/c_h,c_h,c_h], "
                         "gn_w/gn_b [H,d])")
    s = _launch_stream(q.device, stream)
    if out is None:
        # allocated on the launch stream: the caching allocator then never hands
        # its memory to other work while the kernel may still write it
        with torch.cuda.stream(s):
            out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous CUDA tensor like q")
    cfg = make_config(B, H, T, d, c_q, c_k, c_h, kq_place, head_place,
                      I.F32 if q.dtype == torch.float32 else I.BF16, gn_eps, depth_scale)
    if gate is None:
        rc = lib.mta_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), theta_kq.data_ptr(),
                             theta_head.data_ptr(), gn_w.data_ptr(), gn_b.data_ptr(), ctypes.byref(cfg),
                             out.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    else:
        rc = lib.mta_forward_gated(q.data_ptr(), k.data_ptr(), v.data_ptr(), theta_kq.data_ptr(),
                                   theta_head.data_ptr(), gn_w.data_ptr(), gn_b.data_ptr(),
                                   gate.data_ptr(), ctypes.byref(cfg), out.data_ptr(),
                                   ctypes.c_void_p(s.cuda_stream))
    if rc != MTA_OK:
        raise MTAError(rc, status_string(rc))
    return out


GRAD_NAMES = ("q", "k", "v", "theta_kq", "theta_head", "gn_w", "gn_b", "gate")


def backward(q, k, v, theta_kq, theta_head, gn_w, gn_b, dout, *, c_q: int, c_k: int, c_h: int,
             kq_place: int = I.PRE, head_place: int = I.POST, gn_eps: float = 1e-5, depth_scale: float = 1.0,
             gate: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None,
             noalloc: bool = False, workspace_bytes: Optional[int] = None) -> Dict:
    """Gradients of ``forward`` (any placement) through
    ``mta_backward``: returns float32 CUDA tensors keyed q, k, v, theta_kq,
    theta_head, gn_w, gn_b (and gate).  ``dout`` is dL/dout in the input dtype.
    Allocates the outputs and the workspace with torch (the library allocates
    nothing).  With ``noalloc`` the call goes to ``mta_backward_noalloc``, whose
    workspace is the library's own device scratch array (no workspace tensor).
    ``workspace_bytes`` overrides the workspace size the library asks for (the
    map form accepts less and runs more chunks)."""
    lib = load()
    B, H, T, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor like q")
    for name, t in (("theta_kq", theta_kq), ("theta_head", theta_head), ("gn_w", gn_w), ("gn_b", gn_b)):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 CUDA tensor")
    cfg = make_config(B, H, T, d, c_q, c_k, c_h, kq_place, head_place,
                      I.F32 if q.dtype == torch.float32 else I.BF16, gn_eps, depth_scale)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    s = _launch_stream(dev, stream)
    nbytes = int(lib.mta_backward_workspace_size(ctypes.byref(cfg))) if workspace_bytes is None else workspace_bytes
    # outputs and workspace are allocated on the launch stream, so that the
    # caching allocator does not reuse the workspace (freed on return) for other
    # work while the kernels on that stream may still use it
    with torch.cuda.stream(s):
        g = {"q": torch.empty(q.shape, **f32), "k": torch.empty(q.shape, **f32),
             "v": torch.empty(q.shape, **f32), "theta_kq": torch.empty(theta_kq.shape, **f32),
             "theta_head": torch.empty(theta_head.shape, **f32), "gn_w": torch.empty(gn_w.shape, **f32),
             "gn_b": torch.empty(gn_b.shape, **f32)}
        if gate is not None:
            g["gate"] = torch.empty(gate.shape, **f32)
        ws = None if noalloc else torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    ptr = lambda t: t.data_ptr() if t is not None else None
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), theta_kq.data_ptr(), theta_head.data_ptr(),
            gn_w.data_ptr(), gn_b.data_ptr(), ptr(gate), dout.data_ptr(), ctypes.byref(cfg),
            g["q"].data_ptr(), g["k"].data_ptr(), g["v"].data_ptr(), g["theta_kq"].data_ptr(),
            g["theta_head"].data_ptr(), g["gn_w"].data_ptr(), g["gn_b"].data_ptr(), ptr(g.get("gate")))
    if noalloc:
        rc = lib.mta_backward_noalloc(*args, ctypes.c_void_p(s.cuda_stream))
    else:
        rc = lib.mta_backward(*args, ws.data_ptr(), ws.numel(), ctypes.c_void_p(s.cuda_stream))
    if rc != MTA_OK:
        raise MTAError(rc, status_string(rc))
    return g


def backward_cfg(cfg: I.MTAConfig, inp: Dict[str, torch.Tensor], dout: torch.Tensor, stream=None,
                 noalloc: bool = False, workspace_bytes: Optional[int] = None) -> Dict:
    return backward(inp["q"], inp["k"], inp["v"], inp["theta_kq"], inp["theta_head"], inp["gn_w"], inp["gn_b"],
                    dout, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq_place=cfg.kq_place, head_place=cfg.head_place,
                    gn_eps=cfg.gn_eps, depth_scale=cfg.depth_scale, gate=inp.get("gate"), stream=stream,
                    noalloc=noalloc, workspace_bytes=workspace_bytes)


def backward_kernel_name(cfg: I.MTAConfig) -> Optional[str]:
    """Which backward ``mta_backward`` runs for a workload configuration."""
    c = make_config(cfg.B, cfg.H, cfg.T, cfg.d, cfg.c_q, cfg.c_k, cfg.c_h, cfg.kq_place, cfg.head_place,
                    I.F32 if cfg.dtype == "f32" else I.BF16, cfg.gn_eps, cfg.depth_scale)
    r = load().mta_backward_kernel_name(ctypes.byref(c))
    return r.decode() if r else None


def forward_layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gn_w: torch.Tensor, gn_b: torch.Tensor,
                  *, c_h: int, c_q: int = 1, c_k: int = 1, c_q2: int = 1, c_k2: int = 1, exact: bool = False,
                  gn_eps: float = 1e-5, depth_scale: float = 1.0, gate: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None,
                  **kernels) -> torch.Tensor:
    """The general MTA layer through ``mta_forward_layer``.  ``kernels``: any of
    kq_pre [H,c_q,c_k], head_pre, head_post, head_post2 [H/c_h,c_h,c_h], conv3d
    [H/c_h,c_h,c_h,c_q,c_k], kq_post [H,c_q2,c_k2] (float32 CUDA tensors; absent
    or None = stage absent).  Asynchronous on ``stream``."""
    lib = load()
    unknown = set(kernels) - set(LAYER_KERNELS)
    if unknown:
        raise ValueError(f"unknown layer stages {sorted(unknown)}")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must be [B, H, T, d] tensors of one dtype")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q, k, v must be float32 or bfloat16")
    B, H, T, d = q.shape
    G = H // max(c_h, 1)
    shapes = {"kq_pre": (H, c_q, c_k), "head_pre": (G, c_h, c_h), "conv3d": (G, c_h, c_h, c_q, c_k),
              "head_post": (G, c_h, c_h), "kq_post": (H, c_q2, c_k2), "head_post2": (G, c_h, c_h),
              "gn_w": (H, d), "gn_b": (H, d), "gate": (H,)}
    tens = {n: t for n, t in kernels.items() if t is not None}
    tens.update(gn_w=gn_w, gn_b=gn_b)
    if gate is not None:
        tens["gate"] = gate
    for name, t in list(tens.items()) + [("q", q), ("k", k), ("v", v)]:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA (HIP) tensor")
        if name in shapes and (t.dtype != torch.float32 or tuple(t.shape) != shapes[name]):
            raise ValueError(f"{name} must be float32 of shape {shapes[name]}")
    s = _launch_stream(q.device, stream)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous CUDA tensor like q")
    lc, lw = _layer_structs(B, H, T, d, I.F32 if q.dtype == torch.float32 else I.BF16, c_h, c_q, c_k, c_q2,
                            c_k2, exact, gn_eps, depth_scale, {n: t.data_ptr() for n, t in tens.items()})
    rc = lib.mta_forward_layer(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(lw), ctypes.byref(lc),
                               out.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    if rc != MTA_OK:
        raise MTAError(rc, status_string(rc))
    return out


def forward_cfg(cfg: I.MTAConfig, inp: Dict[str, torch.Tensor], out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    if cfg.form != "std":
        w = I.layer_weights(cfg, inp)
        return forward_layer(inp["q"], inp["k"], inp["v"], inp["gn_w"], inp["gn_b"], c_h=cfg.c_h, c_q=cfg.c_q,
                             c_k=cfg.c_k, c_q2=max(cfg.c_q2, 1), c_k2=max(cfg.c_k2, 1),
                             exact=w.pop("exact"), gn_eps=cfg.gn_eps, depth_scale=cfg.depth_scale,
                             gate=inp.get("gate"), out=out, stream=stream,
                             **{n: t for n, t in w.items() if n in LAYER_KERNELS})
    return forward(inp["q"], inp["k"], inp["v"], inp["theta_kq"], inp["theta_head"], inp["gn_w"],
                   inp["gn_b"], c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq_place=cfg.kq_place,
                   head_place=cfg.head_place, gn_eps=cfg.gn_eps, depth_scale=cfg.depth_scale,
                   gate=inp.get("gate"), out=out, stream=stream)
