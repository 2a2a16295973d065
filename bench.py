#!/usr/bin/env python3
"""Benchmark of the Qwen-Image-2.1 denoiser step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1024]

One "step" is one ``qi21_step`` call: the target rows of the workload go
through all 32 blocks against the cached prefix (embed -> 32 x [qkv GEMM,
qkrope, attention, O GEMM, rowop, gate/up GEMM + SwiGLU, down GEMM, rowop]
-> final LayerNorm + proj_out), inputs resident in HBM.  The prefix is
prefilled once before the timed region.  Weights are random (seeded,
bf16, N(0, 0.02)) with the full model's shapes; inputs are synthetic.

The FFN input and the SwiGLU hidden are stored in the lo4 form by default
(f16 plus an MX-scaled e2m1 residual, ``--ffn lo4``), a configuration
whose velocity the tests hold to 1e-3 of the oracle, as they do lo8 (an
e4m3 residual) and pair (f16 pairs); ``--ffn f16`` times the pages'
single-f16 design, which misses that bar on these weights.

Prints ONE JSON line: s/step (the metric), TFLOP/s and the fraction of the
f16 MFMA peak (algorithmic FLOP of the method: the residual products of
the lo8 form are not counted), the dominant kernel's roofline (gate/up
GEMM, timed with HIP events on the launch stream inside the timed region,
around a sample of its launches: one in every ``--event-every``),
every site's MFMA fraction from a separate profiled pass after the timed
region, and the CPU oracle's time on a bounded sample of the same
workload.

This module also holds the GPU-side workload builders the GPU tests use.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import inputs  # noqa: E402
from inputs.configs import (BLOCK_NAMES, CONFIGS, MOD_SIGMA, NORM_SIGMA, ROW_SIGMA,  # noqa: E402
                            TID_FINAL_SCALE, TID_IMG_IN, TID_MODS, TID_MODS0, TID_PREFIX_X,
                            TID_PROJ_OUT, TID_TOK, W_SIGMA, block_tid)

PEAK_F16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
PAGES_STEP_S = {"512": 0.234, "1024": 1.036, "2048": 5.87, "cond": 1.18}  # RTX PRO 4000 via Vulkan (context)


# ───────────────────────────── workload builders ─────────────────────────────

def geom_of(spec):
    from diffusion_transformer_denoiser_qi21_amd import qi21 as Q
    return Q.qi21_geom(hidden=spec.dim, heads=spec.heads, head_dim=spec.head_dim, inter=spec.inter,
                       in_ch=spec.in_ch, eps=spec.eps)


def build_model(spec, opt=None, device="cuda", time_path=False, txt_in=False, torch_alloc=True):
    """A qi21 model holding the seeded synthetic weights of ``spec`` (and,
    with ``time_path`` / ``txt_in``, those of the time path / text front).
    With ``torch_alloc`` (and no hook already in ``opt``) the library takes
    its device memory from torch's caching allocator."""
    import torch
    from diffusion_transformer_denoiser_qi21_amd import qi21 as Q

    if torch_alloc:
        opt = Q.qi21_default_options() if opt is None else opt
        if not opt.alloc:
            Q.DeviceAllocator(device).install(opt)

    s = spec.seed
    img_in = inputs.device_tensor(s, TID_IMG_IN, (spec.dim, spec.in_ch), W_SIGMA, bf16=spec.bf16, device=device).float()
    proj_out = inputs.device_tensor(s, TID_PROJ_OUT, (spec.in_ch, spec.dim), W_SIGMA, bf16=spec.bf16,
                                    device=device).float()
    m = Q.qi21_model_create(geom_of(spec), opt, spec.layers, img_in, proj_out)
    for l in range(spec.layers):
        ws = []
        for j, (name, shape) in enumerate(zip(BLOCK_NAMES, spec.block_shapes())):
            if name.startswith("norm"):
                ws.append(inputs.device_tensor(s, block_tid(l, j), shape, NORM_SIGMA, mean=1.0, device=device))
            else:
                ws.append(inputs.device_tensor(s, block_tid(l, j), shape, W_SIGMA, bf16=spec.bf16, device=device))
        Q.qi21_model_set_block(m, l, None, ws[:7], ws[7], ws[8])
        del ws
    if time_path:
        from inputs.configs import TEMB_IN, TID_MODULATION, TID_NORM_OUT, TID_T_LIN1, TID_T_LIN2
        d = spec.dim
        tw = [inputs.device_tensor(s, tid, shape, W_SIGMA, bf16=spec.bf16, device=device)
              for tid, shape in ((TID_T_LIN1, (d, TEMB_IN)), (TID_T_LIN2, (d, d)), (TID_MODULATION, (4 * d, d)),
                                 (TID_NORM_OUT, (d, d)))]
        Q.qi21_model_set_time(m, None, *tw)
        del tw
    if txt_in:
        from inputs.configs import TID_TXT_IN1, TID_TXT_IN2, TID_TXT_NORM
        d = spec.dim
        Q.qi21_model_set_txt_in(m, d, None, inputs.device_tensor(s, TID_TXT_NORM, (d,), NORM_SIGMA, device=device),
                                inputs.device_tensor(s, TID_TXT_IN1, (d, d), W_SIGMA, bf16=spec.bf16, device=device),
                                inputs.device_tensor(s, TID_TXT_IN2, (d, d), W_SIGMA, bf16=spec.bf16, device=device))
    torch.cuda.synchronize()
    return m


def workload_tensors(w, prefix=0, device="cuda"):
    """Device inputs of workload ``w`` (prefix ``prefix``): prefix rows, RoPE
    tables and visibility from the library's layout helper, modulation,
    tokens and final scale."""
    import torch
    from diffusion_transformer_denoiser_qi21_amd import qi21 as Q

    spec = w.model
    segs = w.layout(prefix)
    t = Q.qi21_layout_tables(segs, tuple(spec.axes), spec.theta)
    lp, n = t["lp"], t["n"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
    d = {
        "lp": lp, "n": n,
        "x": inputs.device_tensor(w.prefix_seed(prefix), TID_PREFIX_X, (lp, spec.dim), ROW_SIGMA, device=device),
        "vis": dev(t["vis"].view(np.int32)),
        "cos_p": dev(t["cos_p"]), "sin_p": dev(t["sin_p"]), "cos_t": dev(t["cos_t"]), "sin_t": dev(t["sin_t"]),
        "mods0": inputs.device_tensor(spec.seed, TID_MODS0, (4 * spec.dim,), MOD_SIGMA, device=device),
        "tok": inputs.device_tensor(w.seed, TID_TOK, (n, spec.in_ch), ROW_SIGMA, device=device),
        "mods": inputs.device_tensor(w.seed, TID_MODS, (4 * spec.dim,), MOD_SIGMA, device=device),
        "fs": 1.0 + inputs.device_tensor(w.seed, TID_FINAL_SCALE, (spec.dim,), MOD_SIGMA, device=device),
    }
    return d


def prefill(m, key, d):
    from diffusion_transformer_denoiser_qi21_amd import qi21 as Q
    Q.qi21_prefill(m, key, d["lp"], d["n"], d["x"], d["cos_p"], d["sin_p"], d["cos_t"], d["sin_t"], d["vis"],
                   d["mods0"])


def step_flops(spec, n, lp, layers=None):
    """Algorithmic FLOP of one step: the four GEMM sites, attention over
    lp + n keys, embed and final (2 FLOP per multiply-add)."""
    h, i, L = spec.dim, spec.inter, spec.layers if layers is None else layers
    gemm = 2.0 * n * (3 * h * h + h * h + 2 * h * i + i * h) * L
    attn = 4.0 * n * (lp + n) * h * L
    io = 4.0 * n * spec.in_ch * h
    return gemm + attn + io, gemm, attn


# ───────────────────────────── CPU baseline ─────────────────────────────

def cpu_baseline(w, min_s=10.0):
    """The oracle as it stands, on a bounded sample of the same workload:
    blocks of the step (all target rows against all keys) timed one after
    the other until at least ``min_s`` seconds of host work, plus embed and
    final, scaled to the full block count."""
    from oracle import SynthModel, workload_inputs
    from oracle import qi21_oracle as O

    spec = w.model
    model = SynthModel(spec, cache_layers=1)
    d = workload_inputs(w)
    lay = O.Layout(w.layout())
    lp, n = lay.prefix_len, lay.target_len
    g = model.geom
    nmax = min(3, spec.layers)
    pre = O.prefill(model, d["x_prefix"], lay, layers=nmax)  # the sample's prefix K/V (not timed)
    every = np.full(n, lp + n, np.int64)
    blocks_done, t_blocks = 0, 0.0
    t0 = time.perf_counter()
    x = O.embed_image(d["tok"], model.img_in)
    t_io = time.perf_counter() - t0
    while blocks_done < nmax and t_blocks < min_s:
        blk = model.block(blocks_done)  # weights regenerated outside the timed region
        t0 = time.perf_counter()
        x, _ = O.block(blk, x, d["mods"], pre.rope_t, (pre.k[blocks_done], pre.v[blocks_done]), every, g)
        t_blocks += time.perf_counter() - t0
        blocks_done += 1
    t0 = time.perf_counter()
    v = O.final_layer(x, d["final_scale"], model.proj_out, g.eps)
    t_io += time.perf_counter() - t0
    est = t_blocks / blocks_done * spec.layers + t_io
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 0) for i in info] + [1])
    except Exception:
        pass
    assert np.all(np.isfinite(v))
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": est, "unit": "s/step", "cores": threads, "cpu_model": cpu, "kind": "oracle",
            "sample": f"{blocks_done} of {spec.layers} blocks of the {w.name} step ({n} target rows vs {lp + n} keys) "
                      f"timed {t_blocks:.1f} s on the host, plus embed and final {t_io:.2f} s; blocks scaled "
                      f"x{spec.layers / blocks_done:.2f}"}


def recorded_traffic(config: str, ffn: str):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter record of this FFN form, or None if none matches this
    workload or any source of the kernel changed since the counters were
    taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"gate_up_gemm_1024_{ffn}_traffic.json")
    if config != "1024" or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    srcs = rec.get("kernel_sources") or {rec["kernel_source"]: rec["kernel_source_sha1"]}
    for src, sha in srcs.items():
        if hashlib.sha1(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != sha:
            return None
    return rec["traffic_bytes_per_launch"]


def copy_calibration(gib: int = 1, reps: int = 5) -> int:
    """A plain device-to-device copy of a known size, run under rocprofv3
    --pmc FETCH_SIZE / WRITE_SIZE to scale those counters to bytes."""
    import torch

    n = gib << 28  # float32 elements
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "reps": reps}))
    return 0


def gemm_vs_hipblaslt(reps: int = 12) -> int:
    """The 256 x 256 GEMM of the step's large sites against hipBLASLt
    (torch.matmul) on the same f16 operands, f16 out: one JSON line per
    shape with both medians (HIP events, interleaved) and the largest
    elementwise difference.  Context for the GEMM roofline, not a step."""
    import torch
    from diffusion_transformer_denoiser_qi21_amd import qi21 as Q

    torch.manual_seed(0)
    M, H, I = 4096, 4096, 12288
    for name, N, K in (("gate/up", 2 * I, H), ("down", H, I), ("O", H, H), ("N 24576, K 12288", 2 * I, I)):
        A = torch.randn(M, K, device="cuda").half()
        W = (torch.randn(N, K, device="cuda") * 0.02).half()
        ref = torch.empty(M, N, device="cuda", dtype=torch.half)
        out = torch.empty(M, N, device="cuda", dtype=torch.half)
        fns = {"hipblaslt": lambda: torch.matmul(A, W.t(), out=ref),
               "qi21": lambda: Q.qi21_op_gemm(Q.QI21_EPI_F16, M, N, K, A, K, W, out, N, tile=0)}
        for f in fns.values():
            for _ in range(3):
                f()
        torch.cuda.synchronize()
        diff = (out.float() - ref.float()).abs().max().item()
        ts = {k: [] for k in fns}
        for _ in range(reps):
            for k, f in fns.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(4):
                    f()
                e1.record()
                torch.cuda.synchronize()
                ts[k].append(e0.elapsed_time(e1) / 4)
        flop = 2.0 * M * N * K
        row = {"shape": name, "M": M, "N": N, "K": K, "max_abs_diff": diff}
        for k, v in ts.items():
            med = sorted(v)[len(v) // 2]
            row[k] = {"median_us": round(med * 1e3, 1), "tflops": round(flop / med / 1e9, 1),
                      "frac": round(flop / med / 1e9 / PEAK_F16_TFLOPS, 4)}
        print(json.dumps(row), flush=True)
    return 0


# ───────────────────────────── main ─────────────────────────────

def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="1024", choices=sorted(k for k in CONFIGS if k != "tiny"))
    ap.add_argument("--ffn", default="lo4", choices=("lo4", "lo8", "pair", "f16"),
                    help="storage of the FFN input and hidden (lo4, the default: f16 + MX-scaled e2m1 residual; "
                         "lo8: f16 + scaled e4m3 residual)")
    ap.add_argument("--site-steps", type=int, default=3,
                    help="steps of the untimed pass that times every site with HIP events")
    ap.add_argument("--event-every", type=int, default=7,
                    help="in the timed region, bracket one gate/up launch in this many with HIP events (an event "
                         "pair delays the launches around it by a few microseconds; 7 is coprime to the 32 "
                         "blocks, so the sample walks every block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (the scale for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--gemm-vs-hipblaslt", action="store_true",
                    help="only time the large-site GEMM against hipBLASLt (torch.matmul) at the step's shapes")
    args = ap.parse_args(argv)
    if args.copy_calibration:
        return copy_calibration()
    if args.gemm_vs_hipblaslt:
        return gemm_vs_hipblaslt()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus above 1 is not supported "
                                   "(a step sharded by target rows over several GPUs is not built)"}))
        return 2

    import torch
    from diffusion_transformer_denoiser_qi21_amd import qi21 as Q

    w = CONFIGS[args.config]
    spec = w.model
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    t_build = time.perf_counter()
    opt = Q.qi21_default_options()
    opt.ffn_mode = {"f16": Q.QI21_FFN_F16, "pair": Q.QI21_FFN_PAIR, "lo8": Q.QI21_FFN_LO8,
                    "lo4": Q.QI21_FFN_LO4}[args.ffn]
    m = build_model(spec, opt)
    t_build = time.perf_counter() - t_build
    nprog = len(w.prefixes)
    ds = [workload_tensors(w, p) for p in range(nprog)]
    t_pre = time.perf_counter()
    for p in range(nprog):
        prefill(m, 100 + p, ds[p])
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t_pre
    n, lp = ds[0]["n"], ds[0]["lp"]
    outs = [torch.empty(n, spec.in_ch, device=dev) for _ in range(nprog)]
    stream = torch.cuda.current_stream()

    def one_step():
        if nprog == 1:
            Q.qi21_step(m, 100, ds[0]["tok"], ds[0]["mods"], ds[0]["fs"], outs[0])
        else:
            Q.qi21_step_batch(m, [100 + p for p in range(nprog)], [d["tok"] for d in ds], ds[0]["mods"],
                              ds[0]["fs"], outs)

    for _ in range(args.warmup):
        one_step()
    Q.qi21_profile_read(m)
    # the timed region: a sample of the dominant kernel's (gate/up GEMM)
    # launches is bracketed by HIP events on the launch stream inside the
    # library
    Q.qi21_set_profile(m, 1 << 4)
    Q.qi21_set_profile_every(m, args.event_every)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_cls, n_cls = Q.qi21_profile_read(m)
    # every site's launches bracketed by events, after the timed region
    site_ms, site_n = None, None
    if args.site_steps > 0:
        Q.qi21_set_profile(m, (1 << 0) | (1 << 2) | (1 << 3) | (1 << 4) | (1 << 5))
        Q.qi21_set_profile_every(m, 1)
        for _ in range(args.site_steps):
            one_step()
        torch.cuda.synchronize()
        site_ms, site_n = Q.qi21_profile_read(m)
    Q.qi21_set_profile(m, 0)
    sec = elapsed / args.steps
    flops = sum(step_flops(spec, d["n"], d["lp"])[0] for d in ds)
    _, gemm_f, attn_f = step_flops(spec, n, lp)
    tflops = flops / sec / 1e12
    w13_launch_ms = ms_cls[4] / max(1, n_cls[4])
    rows_total = sum(d["n"] for d in ds)
    w13_flop = 2.0 * rows_total * 2 * spec.inter * spec.dim
    w13_tf = w13_flop / (w13_launch_ms / 1e3) / 1e12 if w13_launch_ms > 0 else 0.0
    sites = None
    if site_ms is not None:
        h, i = spec.dim, spec.inter
        keys_rows = sum(d["n"] * (d["lp"] + d["n"]) for d in ds)
        per_launch = {  # algorithmic FLOP of one launch (one block) of each site
            "qkv": (0, 2.0 * rows_total * 3 * h * h), "attention": (2, 4.0 * keys_rows * h),
            "o": (3, 2.0 * rows_total * h * h), "gate_up": (4, 2.0 * rows_total * 2 * i * h),
            "down": (5, 2.0 * rows_total * i * h)}
        sites = {}
        g_ms = g_fl = 0.0
        for name, (c, fl) in per_launch.items():
            if site_n[c] == 0:
                continue
            ms = site_ms[c] / site_n[c]
            tf = fl / (ms / 1e3) / 1e12
            sites[name] = {"launch_ms": ms, "tflops": tf, "frac": tf / PEAK_F16_TFLOPS, "launches": int(site_n[c])}
            if name != "attention":
                g_ms += site_ms[c]
                g_fl += fl * site_n[c]
        if g_ms > 0:
            tf = g_fl / (g_ms / 1e3) / 1e12
            sites["all_gemms"] = {"ms_per_step": g_ms / args.site_steps, "tflops": tf, "frac": tf / PEAK_F16_TFLOPS}
        sites["note"] = (f"HIP events around every launch of each site over {args.site_steps} untimed steps after the "
                         "timed region; algorithmic FLOP (the residual forms' extra products not counted)")
    # the residual forms run their FFN GEMMs over 1.25x (lo4: fp4 MFMA at
    # four times the f16 rate) or 1.5x (lo8: fp8 at twice) their K in MFMA
    # cycles, the pair form over 2x: the fraction of the peak of that
    # instruction mix, for context
    mix = {"lo4": 1.25, "lo8": 1.5, "pair": 2.0, "f16": 1.0}[args.ffn]
    line = {
        "metric": "denoiser step s/call + TFLOP/s (% f16 MFMA peak) at 1024^2, 32 blocks",
        "value": sec,
        "unit": "s/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": (sec / PAGES_STEP_S[args.config]) if (args.config in PAGES_STEP_S and nprog == 1) else None,
        "dtype": {"lo4": "f16+e2m1", "lo8": "f16+e4m3", "pair": "f16", "f16": "f16"}[args.ffn],
        "data": "synthetic (seeded N(0,0.02) bf16 weights of the full 32-block dim-4096 model; N(0,1) rows)",
        "config": {"workload": w.note, "blocks": spec.layers, "dim": spec.dim, "heads": spec.heads,
                   "mlp_hidden": spec.inter, "target_rows": rows_total, "prefix_rows": lp, "programs": nprog,
                   "ffn_storage": args.ffn},
        "tflops_per_s": tflops,
        "pct_f16_peak": 100.0 * tflops / PEAK_F16_TFLOPS,
        "step_tflop": flops / 1e12,
        "roofline": {"bound": "mfma", "kernel": "gate/up GEMM + SwiGLU", "achieved": w13_tf,
                     "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": w13_tf / PEAK_F16_TFLOPS,
                     "traffic": recorded_traffic(args.config, args.ffn), "launch_ms": w13_launch_ms,
                     "launches": int(n_cls[4]), "launches_sampled_one_in": args.event_every,
                     "algorithmic_flop": w13_flop,
                     "mfma_mix_frac": w13_tf * mix / PEAK_F16_TFLOPS},
        "sites": sites,
        "device": props.name,
        "build_s": round(t_build, 1),
        "prefill_s": round(t_pre, 3),
    }
    if not args.no_cpu_baseline:
        try:
            cb = cpu_baseline(w)
            line["cpu_baseline"] = cb
        except Exception as e:  # the CPU leg never hides the GPU result
            line["cpu_baseline"] = {"error": repr(e)}
    Q.qi21_model_destroy(m)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
