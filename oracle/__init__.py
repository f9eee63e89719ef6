"""CPU oracle for the Multi-Token Attention forward (test infrastructure).

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it; the
two share no code.

The arithmetic lives in ``mta_oracle.c`` (plain C, float64), which follows the
page "Multi-Token Attention — Paper Graph", section 3.4, step by step.  This
module only builds that file with gcc and marshals arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mta_oracle.c")
LIB = os.path.join(HERE, "libmta_oracle.so")

_lib = None


def build(out: str = LIB, mutant: int = 0, force: bool = True) -> str:
    """Compile the oracle with gcc.  ``mutant`` > 0 plants one of the numbered
    mistakes (used only by the mutation test of the pins)."""
    if not force and os.path.exists(out):
        return out
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC",
           f"-DORACLE_MUTANT={int(mutant)}", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    D = ctypes.POINTER(ctypes.c_double)
    I = ctypes.c_int
    lib.mta_oracle_forward.argtypes = [D, D, D, D, D, D, D, D,
                                       I, I, I, I, I, I, I, I, I,
                                       ctypes.c_double, ctypes.c_double,
                                       I, I, ctypes.POINTER(ctypes.c_int), I, I, I, D]
    lib.mta_oracle_forward.restype = I
    lib.mta_oracle_stages.argtypes = [D, D, D, D, D, D, D, D,
                                      I, I, I, I, I, I, I, I, I,
                                      ctypes.c_double, ctypes.c_double,
                                      I, I, D, D, D, D, D, D, D, D, D]
    lib.mta_oracle_stages.restype = I
    lib.mta_oracle_layer.argtypes = [D] * 12 + [I] * 10 + [ctypes.c_double, ctypes.c_double] + \
        [I, I, ctypes.POINTER(ctypes.c_int), I, I, I, D]
    lib.mta_oracle_layer.restype = I
    lib.mta_oracle_layer_stages.argtypes = [D] * 12 + [I] * 10 + [ctypes.c_double, ctypes.c_double] + \
        [I, I] + [D] * 10
    lib.mta_oracle_layer_stages.restype = I
    lib.mta_oracle_max_threads.argtypes = []
    lib.mta_oracle_max_threads.restype = I
    return lib


def load(path: Optional[str] = None):
    """Load the built oracle (building it first if nothing is built)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: exact upcast (bf16 and fp32 embed in fp64)
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(load().mta_oracle_max_threads())


def default_threads() -> int:
    """Threads for the oracle: OMP_NUM_THREADS if set, else the CPU count,
    capped at 16 (the CPU share of one GPU on the test machines)."""
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _gate(gate, H):
    if gate is None:
        return None, None
    g = _f64(gate)
    assert g.shape == (H,)
    return g, _p(g)


def forward(q, k, v, theta_kq, theta_head, gn_w, gn_b, *, c_q, c_k, c_h,
            kq_place=0, head_place=1, eps=1e-5, depth_scale=1.0, gate=None,
            rows: Optional[Sequence[int]] = None, units: Optional[Sequence[int]] = None,
            chunk: int = 64, threads: Optional[int] = None, lib=None) -> np.ndarray:
    """The forward in float64.  q, k, v: [B,H,T,d].  ``rows`` = (begin, end)
    output rows, ``units`` = list of b*G+g units; outside them the result holds
    NaN.  Returns a float64 array [B,H,T,d]."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    th, w, gw, gb = _f64(theta_kq), _f64(theta_head), _f64(gn_w), _f64(gn_b)
    B, H, T, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    assert th.shape == (H, c_q, c_k) and w.shape == (H // c_h, c_h, c_h)
    assert gw.shape == (H, d) and gb.shape == (H, d)
    r0, r1 = (0, T) if rows is None else (int(rows[0]), int(rows[1]))
    out = np.full((B, H, T, d), np.nan, dtype=np.float64)
    if units is None:
        up, nu = None, 0
    else:
        ua = (ctypes.c_int * len(units))(*[int(u) for u in units])
        up, nu = ua, len(units)
    nt = threads if threads is not None else default_threads()
    ga, gp = _gate(gate, H)
    rc = lib.mta_oracle_forward(_p(q), _p(k), _p(v), _p(th), _p(w), _p(gw), _p(gb), gp,
                                B, H, T, d, c_q, c_k, c_h, kq_place, head_place,
                                float(eps), float(depth_scale), r0, r1, up, nu,
                                int(chunk), int(nt), _p(out))
    if rc != 0:
        raise ValueError(f"mta_oracle_forward failed with code {rc}")
    return out


def stages(q, k, v, theta_kq, theta_head, gn_w, gn_b, *, c_q, c_k, c_h,
           kq_place=0, head_place=1, eps=1e-5, depth_scale=1.0, gate=None, b=0, g=0,
           lib=None) -> Dict[str, np.ndarray]:
    """Every intermediate map of unit (b, g) over all rows: S (logits), C (the
    map entering the softmax before any head mix), Cmix, P (softmax), P2 (after
    a post-softmax key-query conv), P3 (after a post-softmax head mix), O (A V),
    Y (after GroupNorm x depth scale)."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    th, w, gw, gb = _f64(theta_kq), _f64(theta_head), _f64(gn_w), _f64(gn_b)
    B, H, T, d = q.shape
    mats = {n: np.full((c_h, T, T), np.nan) for n in ("S", "C", "Cmix", "P", "P2", "P3")}
    vecs = {n: np.full((c_h, T, d), np.nan) for n in ("O", "Y")}
    out = np.full((B, H, T, d), np.nan)
    ga, gp = _gate(gate, H)
    rc = lib.mta_oracle_stages(_p(q), _p(k), _p(v), _p(th), _p(w), _p(gw), _p(gb), gp,
                               B, H, T, d, c_q, c_k, c_h, kq_place, head_place,
                               float(eps), float(depth_scale), int(b), int(g),
                               _p(mats["S"]), _p(mats["C"]), _p(mats["Cmix"]),
                               _p(mats["P"]), _p(mats["P2"]), _p(mats["P3"]),
                               _p(vecs["O"]), _p(vecs["Y"]), _p(out))
    if rc != 0:
        raise ValueError(f"mta_oracle_stages failed with code {rc}")
    res = dict(mats)
    res.update(vecs)
    res["out"] = out
    return res


LAYER_KERNELS = ("kq_pre", "head_pre", "conv3d", "head_post", "kq_post", "head_post2")


def layer(q, k, v, gn_w, gn_b, *, c_q, c_k, c_h, c_q2=0, c_k2=0, exact=False, eps=1e-5,
          depth_scale=1.0, gate=None, rows: Optional[Sequence[int]] = None,
          units: Optional[Sequence[int]] = None, chunk: int = 64, threads: Optional[int] = None,
          lib=None, **kernels) -> np.ndarray:
    """The general layer in float64 (``kernels``: any of kq_pre, head_pre,
    conv3d, head_post, kq_post, head_post2; absent or None = stage absent).
    Same row/unit selection and result layout as ``forward``."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    gw, gb = _f64(gn_w), _f64(gn_b)
    B, H, T, d = q.shape
    ks = {n: (_f64(kernels[n]) if kernels.get(n) is not None else None) for n in LAYER_KERNELS}
    unknown = set(kernels) - set(LAYER_KERNELS)
    assert not unknown, unknown
    r0, r1 = (0, T) if rows is None else (int(rows[0]), int(rows[1]))
    out = np.full((B, H, T, d), np.nan, dtype=np.float64)
    if units is None:
        up, nu = None, 0
    else:
        up, nu = (ctypes.c_int * len(units))(*[int(u) for u in units]), len(units)
    nt = threads if threads is not None else default_threads()
    ga, gp = _gate(gate, H)
    ptr = [(_p(ks[n]) if ks[n] is not None else None) for n in LAYER_KERNELS]
    rc = lib.mta_oracle_layer(_p(q), _p(k), _p(v), *ptr, _p(gw), _p(gb), gp, B, H, T, d, c_q, c_k,
                              int(c_q2), int(c_k2), c_h, int(bool(exact)), float(eps), float(depth_scale),
                              r0, r1, up, nu, int(chunk), int(nt), _p(out))
    if rc != 0:
        raise ValueError(f"mta_oracle_layer failed with code {rc}")
    return out


def layer_stages(q, k, v, gn_w, gn_b, *, c_q, c_k, c_h, c_q2=0, c_k2=0, exact=False, eps=1e-5,
                 depth_scale=1.0, gate=None, b=0, g=0, lib=None, **kernels) -> Dict[str, np.ndarray]:
    """Every intermediate map of the layer for unit (b, g) over all rows: S,
    Lc (after the pre-softmax convolution), L (entering the softmax), P, Pa
    (after head_post), P2 (after kq_post and Mask_0), P3 (after head_post2), O, Y."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    gw, gb = _f64(gn_w), _f64(gn_b)
    B, H, T, d = q.shape
    ks = {n: (_f64(kernels[n]) if kernels.get(n) is not None else None) for n in LAYER_KERNELS}
    mats = {n: np.full((c_h, T, T), np.nan) for n in ("S", "Lc", "L", "P", "Pa", "P2", "P3")}
    vecs = {n: np.full((c_h, T, d), np.nan) for n in ("O", "Y")}
    out = np.full((B, H, T, d), np.nan)
    ga, gp = _gate(gate, H)
    ptr = [(_p(ks[n]) if ks[n] is not None else None) for n in LAYER_KERNELS]
    rc = lib.mta_oracle_layer_stages(_p(q), _p(k), _p(v), *ptr, _p(gw), _p(gb), gp, B, H, T, d, c_q, c_k,
                                     int(c_q2), int(c_k2), c_h, int(bool(exact)), float(eps),
                                     float(depth_scale), int(b), int(g),
                                     *[_p(mats[n]) for n in ("S", "Lc", "L", "P", "Pa", "P2", "P3")],
                                     _p(vecs["O"]), _p(vecs["Y"]), _p(out))
    if rc != 0:
        raise ValueError(f"mta_oracle_layer_stages failed with code {rc}")
    res = dict(mats)
    res.update(vecs)
    res["out"] = out
    return res


def forward_cfg(cfg, inp: Dict, **kw) -> np.ndarray:
    """Convenience: the forward of an input configuration (the general layer
    for the 3D-convolution and repeated-convolution forms)."""
    if getattr(cfg, "form", "std") != "std":
        from transformer_attention_variant_amd.inputs import layer_weights
        return layer(inp["q"], inp["k"], inp["v"], inp["gn_w"], inp["gn_b"], c_q=cfg.c_q, c_k=cfg.c_k,
                     c_h=cfg.c_h, eps=cfg.gn_eps, depth_scale=cfg.depth_scale, gate=inp.get("gate"),
                     **layer_weights(cfg, inp), **kw)
    return forward(inp["q"], inp["k"], inp["v"], inp["theta_kq"], inp["theta_head"],
                   inp["gn_w"], inp["gn_b"], c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h,
                   kq_place=cfg.kq_place, head_place=cfg.head_place, eps=cfg.gn_eps,
                   depth_scale=cfg.depth_scale, gate=inp.get("gate"), **kw)


def stages_cfg(cfg, inp: Dict, **kw) -> Dict[str, np.ndarray]:
    return stages(inp["q"], inp["k"], inp["v"], inp["theta_kq"], inp["theta_head"],
                  inp["gn_w"], inp["gn_b"], c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h,
                  kq_place=cfg.kq_place, head_place=cfg.head_place, eps=cfg.gn_eps,
                  depth_scale=cfg.depth_scale, gate=inp.get("gate"), **kw)
