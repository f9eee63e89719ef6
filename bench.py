"""Benchmark of the MTA forward on one MI355X.

One step = one ``mta_forward`` call over one batch of the workload (the whole
hot path: logits, key-query convolution, softmax, head mix, P V, GroupNorm),
inputs resident in HBM.  Default workload: the 4K-context layer with planted
needles (B=2, H=16, T=4096, d=128, c_q=6, c_k=11, c_h=2, bf16).

Prints one JSON line with tokens/s, effective TFLOP/s, the roofline of the
kernel (per-launch duration from HIP events recorded on the launch stream
around every launch of the timed region) and the CPU oracle timed on a bounded
sample of the same workload.  Also reported: the same kernel with a 1x1
key-query kernel (the contraction alone; the difference is the convolution
stage) and the per-launch time when a 512 MiB buffer is written before every
launch (inputs no longer in the last-level cache).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MTA fwd tokens/s & eff. TFLOP/s at T=4096, fraction of MFMA/VALU peak"
PEAK_VALU_TFLOPS = 157.3   # fp32 vector, 256 CU x 4 SIMD x 16 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz
PEAK_MFMA_BF16_TFLOPS = 2500.0
PEAK_MFMA_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
FLUSH_MIB = 512


# the HIP sources each forward kernel is built from (its header chain, its
# instantiation unit and the launch helpers)
KERNEL_SOURCES = {
    "mta_fwd_v4": ["mta_fwd_v4.h", "mta_tiles.h", "mta_fwd_kernel.h", "mta_inst_v4.hip", "mta_launch.h"],
    "mta_fwd_kernel": ["mta_fwd_kernel.h", "mta_inst.inc", "mta_inst_bf16.hip", "mta_inst_f32.hip",
                       "mta_launch.h"],
}


def kernel_sources_hash(kernel: str = "") -> str:
    """Hash of the HIP sources of a kernel (of all of them when the kernel is
    not listed); traffic counters are valid only for the sources they were
    taken on."""
    d = os.path.join(ROOT, "transformer_attention_variant_amd", "csrc")
    files = next((v for k, v in KERNEL_SOURCES.items() if kernel.startswith(k + " ")), None)
    if files is None:
        files = [f for f in sorted(os.listdir(d)) if f.endswith((".h", ".hip", ".inc"))]
    h = hashlib.sha256()
    for f in sorted(files):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def stencil_on_matrix_cores(kname) -> bool:
    """Whether the named kernel runs the key-query stencil on the matrix cores
    (fp16 operands) rather than on the fp32 vector ALUs."""
    return kname is not None and kname.startswith(("mta_fwd_v4", "mta_fwd_rep"))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="needle4k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true",
                    help="skip the 1x1-kernel and cache-flushed timings")
    ap.add_argument("--no-backward", action="store_true", help="skip the timing of mta_backward")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows per (batch, head group) unit in the oracle sample, from the end (0 = all)")
    ap.add_argument("--cpu-units", type=int, default=0, help="units in the oracle sample (0 = all)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB `steps` times "
                         "(calibrates the HBM byte counters) and exit")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPYF_DIR", "COPYW_DIR"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this benchmark and of "
                         "--copy-mb into HBM bytes per launch, update --traffic-file, and exit")
    ap.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters (optional)")
    return ap.parse_args()


def _pmc_avg(d, counter, match):
    """Mean of `counter` (KiB per dispatch) over dispatches whose kernel name
    contains `match`, from a rocprofv3 --pmc csv run directory."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and match in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} samples for '{match}' under {d}")
    return sum(vals) / len(vals), len(vals)


def summarize_pmc(args):
    """HBM traffic per launch of the MTA kernel.  FETCH_SIZE and WRITE_SIZE are
    read per dispatch; each is scaled by the ratio of the known byte count of a
    plain device copy (--copy-mb) to what the same counter reports for it."""
    from transformer_attention_variant_amd import binding
    from transformer_attention_variant_amd import inputs as I
    fdir, wdir, cfdir, cwdir = args.summarize_pmc
    kf, nk = _pmc_avg(fdir, "FETCH_SIZE", "mta_fwd")
    kw, _ = _pmc_avg(wdir, "WRITE_SIZE", "mta_fwd")
    cf, _ = _pmc_avg(cfdir, "FETCH_SIZE", "copyBuffer")
    cw, _ = _pmc_avg(cwdir, "WRITE_SIZE", "copyBuffer")
    copy_kib = args.copy_mb * 1024 if args.copy_mb else 512 * 1024
    sf, sw = copy_kib / cf, copy_kib / cw
    rd, wr = kf * sf * 1024, kw * sw * 1024
    entry = {"bytes_per_launch": int(rd + wr), "read_bytes": int(rd), "write_bytes": int(wr),
             "fetch_kib_raw": kf, "write_kib_raw": kw, "fetch_scale": sf, "write_scale": sw,
             "dispatches": nk, "copy_mib": copy_kib // 1024,
             "sources": kernel_sources_hash(binding.kernel_name(I.CONFIGS[args.config]) or "")}
    db = {}
    if os.path.exists(args.traffic_file):
        db = json.load(open(args.traffic_file))
    db[args.config] = entry
    with open(args.traffic_file, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)
    print(json.dumps({args.config: entry}))


RAMP_S = 0.3  # seconds of untimed warm-up before a timed region


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): the MTA "
              "forward here is a single-GPU kernel; sharding over several GPUs is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from transformer_attention_variant_amd import binding
    from transformer_attention_variant_amd import inputs as I

    if args.copy_mb:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "calls": args.steps}))
        return

    cfg = I.CONFIGS[args.config]
    inp = I.generate(cfg)
    dev = {k: v.cuda() for k, v in inp.items()}
    out = torch.empty_like(dev["q"])
    stream = torch.cuda.current_stream()
    K = args.steps

    def timed(c, d, flush=None):
        """(ms per step over the timed region, mean ms per launch) of K calls
        after the warm-up; with `flush`, that buffer is overwritten before
        every launch (outside the per-launch events)."""
        # W warm-up steps, continued (untimed) until the GPU has run the
        # workload for at least RAMP_S seconds, so that its clock has ramped
        # before the timed region
        t0, n = time.time(), 0
        while n < args.warmup or time.time() - t0 < RAMP_S:
            binding.forward_cfg(c, d, out=out, stream=stream)
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(K):
            if flush is not None:
                flush.fill_(float(i))
            ev[i][0].record(stream)
            binding.forward_cfg(c, d, out=out, stream=stream)
            ev[i][1].record(stream)
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / K, float(np.mean([a.elapsed_time(b) for a, b in ev]))

    ms_step, ms_launch = timed(cfg, dev)
    tokens = cfg.B * cfg.T
    value = tokens / (ms_step / 1e3)

    fl = cfg.alg_flops()
    alu_flops = fl["stencil"] + fl["mix"]
    all_flops = fl["contraction"] + fl["stencil"] + fl["mix"]
    t = ms_launch / 1e3
    mfma_peak = PEAK_MFMA_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_MFMA_F32_TFLOPS
    kname = binding.kernel_name(cfg)
    traffic = None
    if os.path.exists(args.traffic_file):
        try:
            tr = json.load(open(args.traffic_file)).get(cfg.name, {})
            if tr.get("sources") == kernel_sources_hash(kname or ""):
                traffic = tr.get("bytes_per_launch")
        except (ValueError, OSError):
            traffic = None
    # The unit that runs the key-query stencil decides the bound.  Kernels with
    # the matrix-core stencil run all the algorithmic work but the head mix
    # (a few VALU FLOP per logit) on the matrix cores, so everything is priced
    # against the 16-bit matrix-core peak; kernels with the fp32 VALU stencil
    # are bound by the vector ALUs and priced against their fp32 peak (the
    # stencil and the head mix, the work that runs there).
    on_mc = stencil_on_matrix_cores(kname)
    if on_mc:
        roof = {
            "bound": "mfma",
            "achieved": round(all_flops / t / 1e12, 2),
            "peak": mfma_peak,
            "unit": "TFLOP/s",
            "frac": round(all_flops / t / 1e12 / mfma_peak, 4),
            "work": ("4*d (QK^T, PV) + 2*(c_q*c_k + c_q2*c_k2) (both key-query convolutions) + 4*c_h "
                     "(both head mixes) FLOP per causal logit" if cfg.form == "repeat" else
                     "4*d (QK^T, PV) + 2*c_q*c_k*c_h (the 3D kernel) FLOP per causal logit" if cfg.form == "3d" else
                     "4*d (QK^T, PV) + 2*c_q*c_k (stencil) + 2*c_h (head mix) FLOP per causal logit"),
        }
    else:
        roof = {
            "bound": "alu",
            "achieved": round(alu_flops / t / 1e12, 3),
            "peak": PEAK_VALU_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(alu_flops / t / 1e12 / PEAK_VALU_TFLOPS, 4),
            "work": "key-query stencil 2*c_q*c_k + head mix 2*c_h FLOP per causal logit",
        }
    roof.update(traffic=traffic, kernel=kname)
    mfma = {
        "achieved": round(fl["contraction"] / t / 1e12, 2),
        "peak": mfma_peak,
        "unit": "TFLOP/s",
        "frac": round(fl["contraction"] / t / 1e12 / mfma_peak, 4),
        "work": "QK^T + PV, 4*d FLOP per causal logit",
    }
    hbm = {"achieved_GBs": round(cfg.io_bytes() / t / 1e9, 1), "peak_GBs": PEAK_HBM_GBS,
           "bytes": cfg.io_bytes(), "work": "read q,k,v + write out"}

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; stand-in shapes for the pages' workloads)",
        "config": {"workload": cfg.name, "batch": cfg.B, "heads": cfg.H, "seq_len": cfg.T,
                   "head_dim": cfg.d, "c_q": cfg.c_q, "c_k": cfg.c_k, "c_h": cfg.c_h,
                   "kq_place": {I.PRE: "pre", I.POST: "post", I.PRE_EXACT: "exact"}[cfg.kq_place],
                   "form": cfg.form, "c_q2": cfg.c_q2, "c_k2": cfg.c_k2,
                   "head_place": "pre" if cfg.head_place == I.PRE else "post",
                   "needles": cfg.needles, "depth_scale": cfg.depth_scale, "global_batch": cfg.B,
                   "parallelism": "single GPU"},
        "eff_tflops": round(all_flops / t / 1e12, 2),
        "ms_per_launch": round(ms_launch, 4),
        "roofline": roof,
        "mfma": mfma,
        "hbm": hbm,
    }

    if not args.no_stages:
        res["stages"] = stages(cfg, dev, timed, t, torch)
    if not args.no_backward and cfg.form == "std":
        res["backward"] = backward_timing(cfg, dev, args, torch)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args)
    print(json.dumps(res), flush=True)


def backward_timing(cfg, dev, args, torch):
    """mta_backward (all input gradients) on the same inputs and a seeded dout,
    timed like the forward (HIP events around every call on the launch stream;
    the outputs and the workspace are allocated once, outside the timed calls)."""
    import ctypes
    from transformer_attention_variant_amd import binding
    from transformer_attention_variant_amd import inputs as I
    g = torch.Generator().manual_seed(cfg.seed + 17)
    dout = torch.randn((cfg.B, cfg.H, cfg.T, cfg.d), generator=g).to(dev["q"].dtype).cuda()
    stream = torch.cuda.current_stream()
    lib = binding.load()
    c = binding.make_config(cfg.B, cfg.H, cfg.T, cfg.d, cfg.c_q, cfg.c_k, cfg.c_h, cfg.kq_place, cfg.head_place,
                            I.F32 if cfg.dtype == "f32" else I.BF16, cfg.gn_eps, cfg.depth_scale)
    f32 = dict(dtype=torch.float32, device=dev["q"].device)
    outs = [torch.empty(dev["q"].shape, **f32) for _ in range(3)] + \
        [torch.empty(dev[n].shape, **f32) for n in ("theta_kq", "theta_head", "gn_w", "gn_b")]
    dgate = torch.empty(dev["gate"].shape, **f32) if "gate" in dev else None
    nws = int(lib.mta_backward_workspace_size(ctypes.byref(c)))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev["q"].device)
    ptr = lambda t: t.data_ptr() if t is not None else None

    def call():
        rc = lib.mta_backward(dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(),
                              dev["theta_kq"].data_ptr(), dev["theta_head"].data_ptr(), dev["gn_w"].data_ptr(),
                              dev["gn_b"].data_ptr(), ptr(dev.get("gate")), dout.data_ptr(), ctypes.byref(c),
                              *[o.data_ptr() for o in outs], ptr(dgate), ws.data_ptr(), nws,
                              ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"mta_backward failed: {binding.status_string(rc)}")

    for _ in range(max(1, args.warmup // 2)):
        call()
    torch.cuda.synchronize()
    K = max(3, args.steps // 2)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(sum(a.elapsed_time(b) for a, b in ev) / K)
    fl = cfg.alg_flops()
    # algorithmic backward work per causal logit: dP3, dV, dQ, dK (8d), the
    # transposed convolution and the kernel gradient (4 c_q c_k), the head mix (4 c_h)
    n = float(cfg.causal_logits())
    bw = n * (8 * cfg.d + 4 * cfg.c_q * cfg.c_k + 4 * cfg.c_h)
    return {"kernel": binding.backward_kernel_name(cfg),
            "ms_per_call": round(ms, 4), "tokens_per_s": round(cfg.B * cfg.T / (ms / 1e3), 1),
            "alg_tflops": round(bw / (ms / 1e3) / 1e12, 2),
            "alg_work": "8d + 4 c_q c_k + 4 c_h FLOP per causal logit (dP3, dV, dQ, dK; transposed "
                        "convolution and kernel gradient; head mix), recomputation not counted",
            "workspace_bytes": nws, "calls": K}


def stages(cfg, dev, timed, t, torch):
    """The convolution stage, read as the difference to the same kernel with a
    1x1 key-query kernel (the stencil collapses to one tap; same c_h, same
    placement), and the cache-flushed launch time."""
    from transformer_attention_variant_amd import binding
    from transformer_attention_variant_amd import inputs as I
    dv = dev["q"].device
    c11 = I.with_(cfg, name=cfg.name + "_1x1", c_q=1, c_k=1, c_q2=1 if cfg.form == "repeat" else cfg.c_q2,
                  c_k2=1 if cfg.form == "repeat" else cfg.c_k2)
    d11 = dict(dev)
    d11["theta_kq"] = torch.ones((cfg.H, 1, 1), dtype=torch.float32, device=dv)
    if "theta_3d" in dev:  # each output head's own delta
        d11["theta_3d"] = torch.eye(cfg.c_h, device=dv).expand(cfg.groups, cfg.c_h, cfg.c_h)\
            .reshape(cfg.groups, cfg.c_h, cfg.c_h, 1, 1).contiguous()
    if "theta_kq2" in dev:
        d11["theta_kq2"] = torch.ones((cfg.H, 1, 1), dtype=torch.float32, device=dv)
    _, ms11 = timed(c11, d11)
    t11 = ms11 / 1e3
    n = float(cfg.causal_logits())
    # the taps beyond the single one of the 1x1 run (per source head for the 3D kernel)
    taps = {"3d": cfg.c_h * (cfg.c_q * cfg.c_k - 1),
            "repeat": cfg.c_q * cfg.c_k - 1 + cfg.c_q2 * cfg.c_k2 - 1}.get(cfg.form, cfg.c_q * cfg.c_k - 1)
    st_alg = 2.0 * taps * n
    # the difference is the convolution stage only if both runs use the same kernel
    same = binding.kernel_name(c11) == binding.kernel_name(cfg) and t > t11
    conv = (t - t11) if same else None
    flush = torch.empty(FLUSH_MIB * (1 << 18), dtype=torch.float32, device=dev["q"].device)
    _, msf = timed(cfg, dev, flush)
    peak_c = PEAK_MFMA_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_MFMA_F32_TFLOPS
    # the convolution stage against the peak of the unit that runs it: the
    # 16-bit matrix cores (fp16 operands) or the fp32 vector ALUs
    on_mc = stencil_on_matrix_cores(binding.kernel_name(cfg))
    conv_peak = PEAK_MFMA_BF16_TFLOPS if on_mc else PEAK_VALU_TFLOPS
    return {
        "kernel_1x1": binding.kernel_name(c11),
        "ms_per_launch_1x1": round(ms11, 4),
        "contraction_tflops_1x1": round(4 * cfg.d * n / t11 / 1e12, 2),
        "contraction_frac_1x1": round(4 * cfg.d * n / t11 / 1e12 / peak_c, 4),
        "conv_stage_ms": round(conv * 1e3, 4) if same else None,
        "conv_stage_tflops": round(st_alg / conv / 1e12, 2) if same else None,
        "conv_stage_unit": "fp16 matrix cores" if on_mc else "fp32 VALU",
        "conv_stage_peak": conv_peak,
        "conv_stage_frac": round(st_alg / conv / 1e12 / conv_peak, 4) if same else None,
        "conv_work": "2*(c_q*c_k - 1) FLOP per causal logit and convolution (the taps beyond the 1x1 "
                     "run's one; per source head for the 3D kernel), counted once; null when the 1x1 run "
                     "selects another kernel",
        "ms_per_launch_flushed": round(msf, 4),
        "flush": f"{FLUSH_MIB} MiB written before every launch",
    }


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, args):
    """The CPU oracle (float64, literal; untuned) on a bounded sample: the last
    ``cpu_rows`` rows of ``cpu_units`` (batch, head group) units.  Each output
    row costs the same in the oracle (it forms every row over all T keys), so
    the full-workload time is the sample time scaled by rows."""
    import oracle
    U = cfg.B * cfg.groups
    nu = U if args.cpu_units <= 0 else min(U, args.cpu_units)
    rows = cfg.T if args.cpu_rows <= 0 else min(cfg.T, args.cpu_rows)
    units = list(range(nu))
    threads = oracle.default_threads()
    q, k, v = (oracle._f64(inp[n]) for n in ("q", "k", "v"))
    lib = oracle.load()
    t0 = time.perf_counter()
    oracle.forward(q, k, v, inp["theta_kq"], inp["theta_head"], inp["gn_w"], inp["gn_b"], c_q=cfg.c_q,
                   c_k=cfg.c_k, c_h=cfg.c_h, kq_place=cfg.kq_place, head_place=cfg.head_place,
                   eps=cfg.gn_eps, depth_scale=cfg.depth_scale, gate=inp.get("gate"),
                   rows=(cfg.T - rows, cfg.T), units=units,
                   chunk=32, threads=threads, lib=lib)
    dt = time.perf_counter() - t0
    full = dt * (U * cfg.T) / (nu * rows)
    return {"value": round(cfg.B * cfg.T / full, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "threads": threads, "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"{nu} of {U} (batch, head group) units x last {rows} of {cfg.T} rows "
                      f"({nu * rows * cfg.c_h} row-heads) in {dt:.2f} s; scaled by rows to the full "
                      f"workload ({full:.1f} s)"}


if __name__ == "__main__":
    main()
