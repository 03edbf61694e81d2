"""Benchmark: fused LM-head forward + backward throughput on one MI355X.

One step = flh_spans_build + flh_forward + flh_backward over one synthetic packed
batch (inputs resident in HBM).  Prints one JSON line:

  value      tokens/s of the whole step (T * steps / elapsed)
  roofline   the dominant kernel's algorithmic flops per launch / its mean launch
             time (HIP events around each launch on the launch stream), against
             the bf16 dense MFMA peak; `traffic` is the measured HBM bytes per
             launch from the committed rocprofv3 counter summary when it was taken
             on the current kernel source, else null
  cpu_baseline  the fp64 oracle timed on the host cores on a token slice of the
             same workload

Default workload: the stress head at its 50% point (T=262144, H=7168, V=129280,
bf16), the largest workload that fits one GPU; --config 2 runs the Llama-3-8B-like
head (T=16384, H=4096, V=128256, about 45% of tokens active).  The line also carries
the median and minimum step time, the algorithmic bandwidth of the memory-bound
kernels, device clocks before and after, a SHA-256 of the input bytes, and a
secondary measurement of the tiny fp32 workload against the fp32 matrix peak.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2516.6e12     # dense bf16 MFMA, 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP8 = 2 * PEAK_BF16  # dense fp8 MFMA (16x16x128 f8f6f4), 5.03 PFLOP/s
PEAK_FP32_MATRIX = 157.3e12
HBM_PEAK = 8.0e12


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=5)
    p.add_argument("--active-frac", type=float, default=None,
                   help="stress workload point (default: its headline 50%%)")
    p.add_argument("--no-hash", action="store_true", help="skip the SHA-256 of the input bytes")
    p.add_argument("--no-secondary", action="store_true", help="skip the tiny fp32 secondary line")
    p.add_argument("--dtype", choices=["auto", "fp8"], default="auto",
                   help="fp8: the workload's draws as OCP E4M3 codes with per-tensor scales "
                        "(flh_forward_fp8 / flh_backward_fp8); auto: the workload's own dtype")
    p.add_argument("--dense", action="store_true", help="dense fallback (no metadata)")
    p.add_argument("--cpu-tokens", type=int, default=1024, help="oracle slice (0 = skip)")
    p.add_argument("--no-trace", action="store_true")
    p.add_argument("--copy-calib-mib", type=int, default=0,
                   help="run one device copy of this many MiB first (counter calibration)")
    p.add_argument("--skip-dw", action="store_true",
                   help="weight gradient over active token tiles only (FLH_BWD_SKIP_INACTIVE_DW; "
                        "the default keeps it dense)")
    p.add_argument("--skip-fwd", action="store_true",
                   help="forward over active token tiles only (FLH_FWD_SKIP_INACTIVE; the default is "
                        "the dense forward)")
    p.add_argument("--padded-tail", action="store_true",
                   help="probe: the padded-staging baseline of the live-width vocabulary split "
                        "(FLH_BWD_PADDED_TAIL; same results)")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the headline run: backward time of the stress workload at its "
                        "active fractions, fitted against the active-tile fraction")
    return p.parse_args()


def method_work(meta, T):
    """(T_at, T_sp, spans) from the device-built active metadata: tokens in active
    128-token tiles (tile bitmap) and tokens inside spans (span list)."""
    tm = int(meta.tile_m)
    n_tiles = -(-T // tm)
    words = meta.tile_bits.cpu().numpy().view(np.uint32)
    idx = np.arange(n_tiles)
    active = (words[idx >> 5] >> (idx & 31).astype(np.uint32)) & 1
    sizes = np.minimum(tm, T - idx * tm)
    spans = meta.host_spans()
    return int((active * sizes).sum()), int(sum(e - s for s, e in spans)), spans


def sweep(args):
    """Backward time vs active fraction on the stress workload (config 5): one line with
    every point and the least-squares fit t_bwd = alpha + beta (T_at + T_sp) / T."""
    import torch

    from entropy_block_sparse_amd import flh_backward, flh_forward, flh_spans_build, flh_workspace_bytes
    from workloads import get_config, make_mask, make_tensors, make_upstream

    cfg = get_config(5)
    dev = torch.device("cuda:0")
    T, H, V, Ssplit = cfg.T, cfg.H, cfg.V, cfg.vocab_split
    h, W, y = make_tensors(T, H, V, cfg.dtype, cfg.seed, device=dev)
    ws_f = torch.empty(flh_workspace_bytes(1, h.dtype, T, H, V), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(flh_workspace_bytes(2, h.dtype, T, H, V, Ssplit), dtype=torch.uint8, device=dev)
    points = []
    runs = [(f, False) for f in cfg.sweep] + [(1.0, True)]
    for frac, dense in runs:
        mask_np, minfo = make_mask(5, active_frac=frac)
        a_np, b_np = make_upstream(mask_np)
        mask = torch.as_tensor(mask_np).to(dev)
        g_lp, g_ent = torch.as_tensor(a_np).to(dev), torch.as_tensor(b_np).to(dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        t_f, t_b = [], []
        for it in range(args.warmup + args.steps):
            ev[0].record()
            meta = None if dense else flh_spans_build(mask)
            lp, ent, lse = flh_forward(h, W, y, workspace=ws_f, meta=meta,
                                       skip_inactive=args.skip_fwd and not dense)
            ev[1].record()
            flh_backward(h, W, y, lse, ent, g_lp, g_ent, mask, meta, Ssplit, workspace=ws_b,
                         skip_inactive_dw=args.skip_dw)
            ev[2].record()
            torch.cuda.synchronize()
            if it >= args.warmup:
                t_f.append(ev[0].elapsed_time(ev[1]))
                t_b.append(ev[1].elapsed_time(ev[2]))
        T_at, T_sp, spans = method_work(flh_spans_build(mask), T)
        points.append({"active_frac": minfo["active_frac"], "dense_fallback": dense, "spans": len(spans),
                       "T_at128_frac": T_at / T, "T_sp_frac": T_sp / T,
                       "x": (T_at + T_sp) / T, "fwd_ms": float(np.median(t_f)),
                       "bwd_ms": float(np.median(t_b)), "bwd_ms_min": float(np.min(t_b))})
        print(f"[sweep] f={frac} dense={dense}: fwd {points[-1]['fwd_ms']:.1f} ms, "
              f"bwd {points[-1]['bwd_ms']:.1f} ms, x={points[-1]['x']:.3f}", file=sys.stderr, flush=True)
    fit_pts = [p for p in points if not p["dense_fallback"]]
    x = np.array([p["x"] for p in fit_pts])
    t = np.array([p["bwd_ms"] for p in fit_pts])
    A_ = np.stack([np.ones_like(x), x], axis=1)
    (alpha, beta), *_ = np.linalg.lstsq(A_, t, rcond=None)
    pred = alpha + beta * x
    r2 = 1.0 - float(((t - pred) ** 2).sum() / max(((t - t.mean()) ** 2).sum(), 1e-30))
    out = {"metric": "stress-workload backward time vs active-tile fraction", "unit": "ms",
           "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "dtype": cfg.dtype, "data": "synthetic",
           "config": {"workload": cfg.name, "T": T, "H": H, "V": V, "vocab_split": Ssplit,
                      "skip_inactive_dw": bool(args.skip_dw), "skip_inactive_fwd": bool(args.skip_fwd)},
           "points": points,
           "fit": {"model": "t_bwd = alpha + beta * (T_at + T_sp) / T", "alpha_ms": float(alpha),
                   "beta_ms": float(beta), "r2": r2}}
    print(json.dumps(out))


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "entropy_block_sparse_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def workload_label(cfg, frac, fp8=False):
    """Name of a workload point: the config name, plus the active fraction for the
    stress workload (whose points differ only in the mask), plus the input dtype when
    it is fp8."""
    name = cfg.name if cfg.cid != 5 else f"{cfg.name} active={frac:.2f}"
    return name + (" fp8" if fp8 else "")


def clock_snapshot():
    """Current engine and memory clock levels and the power cap of the GPU(s), read from
    sysfs (no other program is started: this process has initialised the GPU).  None
    where a file is missing."""
    import glob

    def cur(path):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return line.split(":", 1)[1].strip(" *\n")
        except OSError:
            return None
        return None

    cards = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        if not os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
            continue
        cap = None
        for hw in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_cap")):
            try:
                with open(hw) as f:
                    cap = int(f.read().strip()) / 1e6
            except (OSError, ValueError):
                pass
        cards.append({"card": os.path.basename(os.path.dirname(dev)), "sclk": cur(os.path.join(dev, "pp_dpm_sclk")),
                      "mclk": cur(os.path.join(dev, "pp_dpm_mclk")), "power_cap_w": cap})
    if not cards:
        return {"source": "sysfs unavailable"}
    return {"source": "sysfs", "cards": cards[:8]}


def input_sha256(*tensors, chunk=1 << 28):
    """SHA-256 over the raw bytes of device tensors, in order, copied to the host in
    chunks."""
    import torch

    hsh = hashlib.sha256()
    for t in tensors:
        flat = t.contiguous().view(-1).view(torch.uint8) if t.dtype != torch.uint8 else t.contiguous().view(-1)
        for i in range(0, flat.numel(), chunk):
            hsh.update(flat[i:i + chunk].cpu().numpy().tobytes())
    return hsh.hexdigest()


def aux_bytes(name, T, H, V, esz, A, n_spans, n_splits, ld_wt, ld_t, in_esz=None):
    """Algorithmic bytes per launch of the memory-bound kernels (reads + writes).
    esz: element size of the gradients and transposed copies; in_esz: of h and W
    (1 for fp8 codes)."""
    in_esz = in_esz or esz
    n_tiles = -(-T // 128)
    if name == "spans_build":
        return T + 8 * n_spans + 4 * -(-n_tiles // 32) + 8
    if name == "bwd_lists":
        return 4 * -(-n_tiles // 32) + 8 * n_spans + 4 * n_tiles + 8 * (T // 32 + n_spans) + 4 * -(-T // 32)
    if name == "fwd_target_logit":
        return 2 * T * H * in_esz + 8 * T + 4 * T
    if name == "fwd_combine":
        return -(-V // 256) * T * 16 + 4 * T + 12 * T
    if name == "dhidden_finalize":
        return A * H * 4 + T * H * esz + T + 4 * -(-T // 32)
    if name == "transpose":  # the W and h transposes of one backward, per launch on average
        return ((V * H + T * H) * in_esz + (n_splits * H * ld_wt + H * ld_t) * esz) / 2
    return None


def stored_traffic(kernel: str, workload: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    rec = d.get(workload, {}).get(kernel)
    if not rec or rec.get("source_sha") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(h, W, y, mask, a, b, n_tok, scales=None):
    """The fp64 oracle (forward + backward) on the first n_tok tokens, full H and V.
    scales: (scale_h, scale_w) when h and W hold fp8 codes (decoded by the oracle)."""
    import threadpoolctl

    from oracle import fp8 as O8
    from oracle import lmhead as O

    if scales is not None:
        hs = O8.dequantize(h[:n_tok].cpu().numpy(), scales[0])
        Wf = O8.dequantize(W.cpu().numpy(), scales[1])
    else:
        hs = h[:n_tok].float().cpu().numpy().astype(np.float64)
        Wf = W.float().cpu().numpy().astype(np.float64)
    ys = y[:n_tok].cpu().numpy()
    ms = mask[:n_tok]
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    t0 = time.perf_counter()
    O.forward(hs, Wf, ys)
    O.backward(hs, Wf, ys, ms, a[:n_tok], None if b is None else b[:n_tok])
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n_tok} tokens of the workload at full H and V, fp64 numpy "
                      f"forward+backward{' on the decoded fp8 inputs' if scales else ''}, {dt:.2f} s"}


def tiny_fp32_line(torch, dev, steps=50, warmup=5):
    """The tiny fp32 workload (T=512, H=256, V=4096) timed like the headline: tokens/s
    and the method's flops against the fp32 matrix peak (the bf16 peak does not apply)."""
    from entropy_block_sparse_amd import flh_backward, flh_forward, flh_spans_build, flh_workspace_bytes
    from workloads import get_config, make_mask, make_tensors, make_upstream

    cfg = get_config(1)
    T, H, V = cfg.T, cfg.H, cfg.V
    mask_np, _ = make_mask(1)
    h, W, y = make_tensors(T, H, V, cfg.dtype, cfg.seed, device=dev)
    a_np, b_np = make_upstream(mask_np)
    mask = torch.as_tensor(mask_np).to(dev)
    g_lp, g_ent = torch.as_tensor(a_np).to(dev), torch.as_tensor(b_np).to(dev)
    ws_f = torch.empty(flh_workspace_bytes(1, h.dtype, T, H, V), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(flh_workspace_bytes(2, h.dtype, T, H, V, cfg.vocab_split), dtype=torch.uint8, device=dev)

    def step():
        meta = flh_spans_build(mask)
        lp, ent, lse = flh_forward(h, W, y, workspace=ws_f)
        return flh_backward(h, W, y, lse, ent, g_lp, g_ent, mask, meta, cfg.vocab_split, workspace=ws_b)

    for _ in range(warmup):
        step()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / steps
    T_at, T_sp, _ = method_work(flh_spans_build(mask), T)
    F = 2.0 * H * V * (T + T_at + T_sp + T)
    return {"workload": cfg.name, "dtype": "f32", "value": T / (ms * 1e-3), "unit": "tokens/s",
            "ms_per_step": ms, "median_ms": float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])),
            "steps": steps, "frac_fp32_matrix_peak": F / (ms * 1e-3) / PEAK_FP32_MATRIX,
            "note": "launch-latency bound: about 1 GFLOP per pass"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    import torch

    from entropy_block_sparse_amd import (flh_backward, flh_backward_fp8, flh_forward, flh_forward_fp8,
                                          flh_spans_build, flh_workspace_bytes, trace_begin, trace_end)
    from workloads import get_config, make_mask, make_tensors, make_tensors_fp8, make_upstream

    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    frac_req = args.active_frac if args.active_frac is not None else (cfg.target_active if cfg.cid == 5 else None)
    mask_np, minfo = make_mask(cfg.cid, active_frac=frac_req)
    T, H, V, Ssplit = cfg.T, cfg.H, cfg.V, cfg.vocab_split
    fp8 = args.dtype == "fp8"
    if fp8:
        h, s_h, W, s_w, y = make_tensors_fp8(T, H, V, cfg.seed, device=dev)
    else:
        h, W, y = make_tensors(T, H, V, cfg.dtype, cfg.seed, device=dev)
    a_np, b_np = make_upstream(mask_np)
    mask = torch.as_tensor(mask_np).to(dev)
    g_lp = torch.as_tensor(a_np).to(dev)
    g_ent = torch.as_tensor(b_np).to(dev)
    ws_f = torch.empty(flh_workspace_bytes(1, h.dtype, T, H, V), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(flh_workspace_bytes(2, h.dtype, T, H, V, Ssplit), dtype=torch.uint8, device=dev)

    def step():
        meta = None if args.dense else flh_spans_build(mask)
        if fp8:
            lp, ent, lse = flh_forward_fp8(h, s_h, W, s_w, y, workspace=ws_f, meta=meta,
                                           skip_inactive=args.skip_fwd and not args.dense)
            return flh_backward_fp8(h, s_h, W, s_w, y, lse, ent, g_lp, g_ent, mask, meta, Ssplit, workspace=ws_b,
                                    skip_inactive_dw=args.skip_dw)
        lp, ent, lse = flh_forward(h, W, y, workspace=ws_f, meta=meta,
                                   skip_inactive=args.skip_fwd and not args.dense)
        dH, dW = flh_backward(h, W, y, lse, ent, g_lp, g_ent, mask, meta, Ssplit, workspace=ws_b,
                              skip_inactive_dw=args.skip_dw, padded_tail=args.padded_tail)
        return dH, dW

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    clocks_before = clock_snapshot()
    trace = not args.no_trace
    if trace:
        trace_begin(64 * args.steps + 64)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    recs = trace_end(64 * args.steps + 64) if trace else []
    clocks_after = clock_snapshot()

    # ---- algorithmic work of the method ----
    T_at, T_sp, spans = method_work(flh_spans_build(mask), T)
    A = int(mask_np.sum())
    pass_flops = 2.0 * H * V
    F_min = pass_flops * (2 * T + 2 * A)
    T_dw = T_at if (args.skip_dw and not args.dense) else T  # tokens the weight gradient covers
    T_fwd = T_at if (args.skip_fwd and not args.dense) else T  # tokens the forward covers
    F_method = pass_flops * (T_fwd + T_at + T_sp + T_dw) if not args.dense else pass_flops * 4 * T
    peak = PEAK_BF16 if cfg.dtype == "bf16" else PEAK_FP32_MATRIX
    # each contraction's own peak: fp8 inputs run the forward and d-logits on fp8 matrix
    # instructions and the hidden- and weight-gradient products in bf16
    kpeak = {"fwd_logits_softmax": PEAK_FP8 if fp8 else peak, "dlogits": PEAK_FP8 if fp8 else peak,
             "dhidden_spans": peak, "dweight": peak}

    per_kernel = {}
    for name, split, kms in recs:
        d = per_kernel.setdefault(name, {"launches": 0, "ms": 0.0})
        d["launches"] += 1
        d["ms"] += kms
    for d in per_kernel.values():
        d["ms_per_step"] = d["ms"] / args.steps
        d["ms_per_launch"] = d["ms"] / max(1, d["launches"])
    # algorithmic flops per launch of each contraction kernel
    n_splits = -(-V // Ssplit)
    alg = {
        "fwd_logits_softmax": pass_flops * T_fwd,
        "dweight": pass_flops * T_dw / n_splits,
        "dlogits": pass_flops * T_at / n_splits,
        "dhidden_spans": pass_flops * T_sp / n_splits,
    }
    esz = 2 if cfg.dtype == "bf16" else 4
    n_sp = -(-V // Ssplit)
    w_max = min(V, Ssplit)
    pad = lambda n: (-(-n // 64) * 64) + (64 if (-(-n // 64)) % 2 == 0 else 0)  # noqa: E731
    for k, d in per_kernel.items():
        nb = aux_bytes(k, T, H, V, esz, A, len(spans), n_sp, pad(w_max), pad(-(-T // 128) * 128),
                       1 if fp8 else esz)
        if nb is not None and d["ms_per_launch"] > 0:
            d["alg_bytes_per_launch"] = nb
            d["gbps"] = nb / (d["ms_per_launch"] * 1e-3) / 1e9
    roof = None
    if per_kernel:
        dom = max((k for k in per_kernel if k in alg), key=lambda k: per_kernel[k]["ms"])
        achieved = alg[dom] / (per_kernel[dom]["ms_per_launch"] * 1e-3)
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved / 1e12, "peak": kpeak[dom] / 1e12,
                "unit": "TFLOP/s", "frac": achieved / kpeak[dom],
                "traffic": stored_traffic(dom, workload_label(cfg, frac_req or 0.0, fp8))}
        for k in per_kernel:
            if k in alg:
                per_kernel[k]["tflops"] = alg[k] / (per_kernel[k]["ms_per_launch"] * 1e-3) / 1e12
                per_kernel[k]["frac_of_peak"] = per_kernel[k]["tflops"] * 1e12 / kpeak[k]

    sha = None if args.no_hash else input_sha256(h, W, y, mask)
    # fraction of peak of the whole step with every contraction at its own dtype's peak
    t_at_peak = (pass_flops * T_fwd / kpeak["fwd_logits_softmax"] + pass_flops * T_at / kpeak["dlogits"]
                 + pass_flops * T_sp / peak + pass_flops * T_dw / peak) if not args.dense else None
    secondary = None if (args.no_secondary or cfg.cid == 1) else tiny_fp32_line(torch, dev)

    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(h, W, y, mask_np, a_np, b_np, min(args.cpu_tokens, T), (s_h, s_w) if fp8 else None)

    out = {
        "metric": "fused LM-head fwd+bwd tokens/sec at 1 GPU + % of bf16 MFMA peak",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (bf16 gradients)" if fp8 else cfg.dtype,
        "data": "synthetic",
        "config": {"workload": workload_label(cfg, frac_req or 0.0, fp8), "T": T, "H": H, "V": V, "vocab_split": Ssplit,
                   "active_frac": minfo["active_frac"], "mask_seed": minfo["seed"],
                   "dense_fallback": bool(args.dense), "skip_inactive_dw": bool(args.skip_dw),
                   "skip_inactive_fwd": bool(args.skip_fwd), "padded_tail": bool(args.padded_tail)},
        "pct_peak_method": F_method / (ms * 1e-3) / peak,
        "pct_peak_method_per_dtype": (t_at_peak / (ms * 1e-3)) if t_at_peak else None,
        "step_ms": {"mean": ms, "median": float(np.median(step_ms)), "min": float(np.min(step_ms)),
                    "max": float(np.max(step_ms))},
        "active_tokens_per_s": A / (ms * 1e-3),
        "work": {"A": A, "T_at128": int(T_at), "T_sp": int(T_sp), "spans": len(spans),
                 "F_method_tflop": F_method / 1e12, "F_min_tflop": F_min / 1e12,
                 "F_dense_tflop": 4 * pass_flops * T / 1e12,
                 "pct_peak_min": F_min / (ms * 1e-3) / peak},
        "inputs": {"seed": cfg.seed, "mask_seed": minfo["seed"], "sha256_h_W_y_mask": sha},
        "clocks": {"before": clocks_before, "after": clocks_after},
        "secondary": secondary,
        "kernels": per_kernel,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
