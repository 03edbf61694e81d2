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

Default workload: the Llama-3-8B-like head (T=16384, H=4096, V=128256, bf16,
about 45% of tokens active).
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
PEAK_FP32_MATRIX = 157.3e12
HBM_PEAK = 8.0e12


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=2)
    p.add_argument("--active-frac", type=float, default=None, help="stress workload point")
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


def cpu_baseline(h, W, y, mask, a, b, n_tok):
    """The fp64 oracle (forward + backward) on the first n_tok tokens, full H and V."""
    import threadpoolctl

    from oracle import lmhead as O

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
                      f"forward+backward, {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    import torch

    from entropy_block_sparse_amd import (flh_backward, flh_forward, flh_spans_build,
                                          flh_workspace_bytes, trace_begin, trace_end)
    from workloads import get_config, make_mask, make_tensors, make_upstream

    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    mask_np, minfo = make_mask(cfg.cid, active_frac=args.active_frac)
    T, H, V, Ssplit = cfg.T, cfg.H, cfg.V, cfg.vocab_split
    h, W, y = make_tensors(T, H, V, cfg.dtype, cfg.seed, device=dev)
    a_np, b_np = make_upstream(mask_np)
    mask = torch.as_tensor(mask_np).to(dev)
    g_lp = torch.as_tensor(a_np).to(dev)
    g_ent = torch.as_tensor(b_np).to(dev)
    ws_f = torch.empty(flh_workspace_bytes(1, h.dtype, T, H, V), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(flh_workspace_bytes(2, h.dtype, T, H, V, Ssplit), dtype=torch.uint8, device=dev)

    def step():
        meta = None if args.dense else flh_spans_build(mask)
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

    trace = not args.no_trace
    if trace:
        trace_begin(64 * args.steps + 64)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    recs = trace_end(64 * args.steps + 64) if trace else []

    # ---- algorithmic work of the method ----
    T_at, T_sp, spans = method_work(flh_spans_build(mask), T)
    A = int(mask_np.sum())
    pass_flops = 2.0 * H * V
    T_dw = T_at if (args.skip_dw and not args.dense) else T  # tokens the weight gradient covers
    T_fwd = T_at if (args.skip_fwd and not args.dense) else T  # tokens the forward covers
    F_method = pass_flops * (T_fwd + T_at + T_sp + T_dw) if not args.dense else pass_flops * 4 * T
    peak = PEAK_BF16 if cfg.dtype == "bf16" else PEAK_FP32_MATRIX

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
    roof = None
    if per_kernel:
        dom = max((k for k in per_kernel if k in alg), key=lambda k: per_kernel[k]["ms"])
        achieved = alg[dom] / (per_kernel[dom]["ms_per_launch"] * 1e-3)
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": stored_traffic(dom, cfg.name)}
        for k in per_kernel:
            if k in alg:
                per_kernel[k]["tflops"] = alg[k] / (per_kernel[k]["ms_per_launch"] * 1e-3) / 1e12

    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(h, W, y, mask_np, a_np, b_np, min(args.cpu_tokens, T))

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
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": H, "V": V, "vocab_split": Ssplit,
                   "active_frac": minfo["active_frac"], "mask_seed": minfo["seed"],
                   "dense_fallback": bool(args.dense), "skip_inactive_dw": bool(args.skip_dw),
                   "skip_inactive_fwd": bool(args.skip_fwd), "padded_tail": bool(args.padded_tail)},
        "pct_peak_method": F_method / (ms * 1e-3) / peak,
        "work": {"A": A, "T_at128": int(T_at), "T_sp": int(T_sp), "spans": len(spans),
                 "F_method_tflop": F_method / 1e12, "F_dense_tflop": 4 * pass_flops * T / 1e12},
        "kernels": per_kernel,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
