#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer forward on one MI355X.

A step is one full forward of the layer (router -> gating/top-k -> dispatch -> [latent down]
-> grouped SwiGLU experts -> combine [-> norm -> latent up]) over one batch of synthetic
tokens, with inputs and weights resident in HBM. Default workload: the OlmoE-shaped layer
(8192 tokens, d_model 2048, 64 experts, top-8, hidden 1024, bf16, fp32 router).

Printed: one JSON line with tokens/s for the whole layer, the roofline of the dominant stage
(the grouped expert GEMMs, timed with HIP events on the stream they run on), and the CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA (MXFP8 experts)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="olmoe")
    ap.add_argument("--precision", default="bf16", choices=("bf16", "mxfp8"),
                    help="precision of the expert matmuls (mxfp8: block-scaled E4M3 on the fp8 matrix cores)")
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens of the workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mxfp8", action="store_true",
                    help="skip the extra measurement of the same layer with MXFP8 expert matmuls")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the extra measurement of the routed experts' backward")
    ap.add_argument("--stages", action="store_true", help="also time each stage call alone")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the measurement of the achievable matrix-core and copy rates")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times): the reference the HBM "
                         "byte counters are scaled by")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="no GPU: write profiles/expert_gemm_traffic_<workload>.json from four rocprofv3 "
                         "--pmc output folders (FETCH_SIZE and WRITE_SIZE of this bench, then of "
                         "--copy-calibration 256)")
    return ap.parse_args()


GEMM_SOURCES = ("gemm_bf16.hip", "common.hpp")  # the expert GEMM kernels and what they include


def kernel_source_sha256():
    """Hash of the sources the expert GEMM kernels are built from: a counter record taken on
    other sources describes another kernel."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        h.update(name.encode())
        with open(os.path.join(ROOT, "top_routing_grouped_router_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per expert-stage launch from the committed counter record (rocprofv3
    FETCH_SIZE / WRITE_SIZE scaled by a copy calibration), or None when no record exists for
    this workload or the kernel sources changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"expert_gemm_traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_sha256():
        return None
    return rec.get("bytes_per_launch")


def event_time_ms(fn, n, torch):
    """Average GPU time of fn() over n calls, each bracketed by events on the current stream."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / n


def _counter_rows(folder):
    """(kernel name, counter value) per dispatch from a rocprofv3 --pmc csv output folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    with open(files[0]) as f:
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(f)]


def _mean(vals):
    if not vals:
        raise SystemExit("counter record: kernel not found in the profile")
    return sum(vals) / len(vals)


def record_traffic(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib=256):
    """HBM bytes per expert-stage launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the two
    expert GEMM kernels, each scaled by what the same counter reads for a plain device copy of
    copy_mib MiB. Written with the hash of the kernel sources, so that a later change of the
    kernels voids the record."""
    def gemm_kind(name):
        if "gemm_bf16_kernel" not in name:
            return None
        # template arguments after the tile shape: SWIGLU, GATHER, SCATTER, then the output,
        # operand-layout and epilogue options, all off for the two forward GEMMs
        tail = name.split(">", 1)[1] if ">" in name else name
        flags = [t.strip() for t in tail.split(">")[0].split(",")][1:]
        rest = flags[3:]
        if any(f not in ("false", "0") for f in rest):
            return None
        if flags[:3] == ["true", "true", "false"]:
            return "gemm1"
        if flags[:3] == ["false", "false", "true"]:
            return "gemm2"
        return None

    def per_kernel(folder):
        # one stage launch runs each GEMM as up to two kernels (the large tile shape and the
        # small one for remainder rows): average each kernel over its dispatches, then add the
        # kernels of a GEMM
        by_name = {}
        for name, v in _counter_rows(folder):
            kind = gemm_kind(name)
            if kind:
                by_name.setdefault((kind, name), []).append(v)
        out = {"gemm1": 0.0, "gemm2": 0.0}
        for (kind, _), vals in by_name.items():
            out[kind] += _mean(vals)
        if not out["gemm1"] or not out["gemm2"]:
            raise SystemExit("counter record: expert GEMM kernels not found in the profile")
        return out

    def copy_kib(folder):
        vals = sorted((v for name, v in _counter_rows(folder) if "copyBuffer" in name), reverse=True)
        return _mean(vals[:3])

    copied = float(copy_mib << 10)
    cf, cw = copy_kib(copy_fetch_dir), copy_kib(copy_write_dir)
    fetch, write = per_kernel(fetch_dir), per_kernel(write_dir)
    fs, ws = copied / cf, copied / cw
    total = sum(fetch.values()) * fs * 1024 + sum(write.values()) * ws * 1024
    rec = {
        "workload": workload,
        "kernels": "gemm_bf16 GEMM1 (up/gate + SwiGLU, gathered A) + GEMM2 (down, scattered C), "
                   "one launch each per stage",
        "source_sha256": kernel_source_sha256(),
        "source_files": list(GEMM_SOURCES),
        "fetch_size_kib_per_launch": fetch,
        "write_size_kib_per_launch": write,
        "copy_calibration": {"bytes_copied_kib": copied, "fetch_size_kib": cf, "write_size_kib": cw,
                             "fetch_scale": fs, "write_scale": ws},
        "bytes_per_launch": int(round(total)),
    }
    path = os.path.join(ROOT, "profiles", f"expert_gemm_traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def calibration(moe, torch):
    """Achievable matrix-core rates (TFLOP/s: bf16, and the block-scaled FP8 of the MXFP8 experts)
    and HBM copy rate (GB/s of read + write) of this device, each the median of 5 event-timed
    launches of the library's calibration kernels (about 3 ms each)."""
    def loop_rate(run):
        out, _ = run(200)
        t = event_time_ms(lambda: run(200, out), 3, torch)
        iters = max(200, int(200 * 3.0 / max(t, 1e-3)))
        run(iters, out)
        ts = sorted(event_time_ms(lambda: run(iters, out), 1, torch) for _ in range(5))
        return run(iters, out)[1] / (ts[2] / 1e3) / 1e12, iters, ts[2]

    bf16, iters, ms = loop_rate(moe.calibrate_mfma_bf16)
    mx, mx_iters, mx_ms = loop_rate(moe.calibrate_mfma_mxfp8)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    moe.calibrate_copy(src, dst)
    cs = sorted(event_time_ms(lambda: moe.calibrate_copy(src, dst), 1, torch) for _ in range(5))
    del src, dst
    return {"mfma_bf16_tflops": round(bf16, 1), "mfma_loop_iters": iters, "mfma_loop_ms": round(ms, 4),
            "mfma_mxfp8_tflops": round(mx, 1), "mfma_mxfp8_loop_iters": mx_iters,
            "mfma_mxfp8_loop_ms": round(mx_ms, 4),
            "copy_gbs": round(2 * nbytes / (cs[2] / 1e3) / 1e9, 1), "copy_bytes": nbytes,
            "copy_ms": round(cs[2], 4)}


def cpu_baseline(cfg, w, x, n_tokens):
    import numpy as np
    import workloads
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    n = min(n_tokens, x.shape[0])
    xs = workloads.to_numpy_f32(x[:n])
    wo = {k: workloads.to_numpy_f32(v) for k, v in w.items()}
    cfgO = O.MoEConfig.from_dict(cfg)
    t0 = time.perf_counter()
    O.forward(cfgO, wo, xs)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n} tokens of the {x.shape[0]}-token batch, full weights, float64 oracle "
                      f"({dt:.1f} s; {platform.processor() or platform.machine()})"}


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    import top_routing_grouped_router_amd as moe
    import workloads

    name = args.workload
    cfg, w, x = workloads.make_workload(name, device="cuda", expert_precision=args.precision)
    T = x.shape[0]
    E, k, h = cfg["num_experts"], cfg["top_k"], cfg["hidden_size"]
    d, L = cfg["d_model"], cfg["latent_dim"] or 0
    K = L or d
    A = T * k
    layer = moe.MoELayer(cfg, w)
    w = layer.weights  # with the MXFP8 weight copies when the experts run in MXFP8
    y = torch.empty_like(x)

    for _ in range(args.warmup):
        layer(x, out=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer(x, out=y)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    tokens_per_s = T / (ms / 1e3)

    # Dominant stage: the grouped expert GEMMs (tile list, up/gate GEMM + SwiGLU, down GEMM).
    _, r = layer(x, routing=("expert_offsets", "permutation", "expert_weights"))
    z = moe.latent_down(cfg, w, x) if L else x
    offs, perm = r["expert_offsets"], r["permutation"]
    for _ in range(2):
        moe.experts_forward(cfg, w, z, offs, perm)
    gemm_ms = event_time_ms(lambda: moe.experts_forward(cfg, w, z, offs, perm), max(args.steps, 5), torch)
    gemm_flops = 6.0 * A * K * h
    achieved = gemm_flops / (gemm_ms / 1e3) / 1e12
    peak = PEAK_FP8_TFLOPS if args.precision == "mxfp8" else PEAK_BF16_TFLOPS
    layer_flops = 2.0 * T * d * E + gemm_flops + (4.0 * T * d * L if L else 0.0)

    out = {
        "metric": "MoE layer fwd tokens/s + grouped-GEMM % of bf16 MFMA peak, 1xMI355X",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp8 experts, bf16" if args.precision == "mxfp8" else "bf16") if cfg["dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": name, "tokens": T, "d_model": d, "num_experts": E, "top_k": k,
                   "hidden_size": h, "latent_dim": L or None, "gating": cfg["gating_function"],
                   "router": "fp32", "expert_precision": args.precision, "parallelism": "none (1 GPU)"},
        "layer_tflops": round(layer_flops / (ms / 1e3) / 1e12, 2),
        "roofline": {"kernel": "grouped expert GEMMs (up/gate+SwiGLU, down)", "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": recorded_traffic(name) if args.precision == "bf16" else None,
                     "stage_ms": round(gemm_ms, 4), "flops_per_launch": gemm_flops},
    }
    if args.precision == "bf16" and cfg["dtype"] == "bf16" and not args.no_mxfp8:
        # The same layer with the expert matmuls in MXFP8 (block-scaled E4M3; weights quantised
        # once, outside the timed region): an extra record, not the headline.
        cfg8 = dict(cfg, expert_precision="mxfp8")
        layer8 = moe.MoELayer(cfg8, w)
        for _ in range(args.warmup):
            layer8(x, out=y)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            layer8(x, out=y)
        torch.cuda.synchronize()
        ms8 = (time.perf_counter() - t0) * 1e3 / args.steps
        w8 = layer8.weights
        for _ in range(2):
            moe.experts_forward(cfg8, w8, z, offs, perm)
        g8 = event_time_ms(lambda: moe.experts_forward(cfg8, w8, z, offs, perm), max(args.steps, 5), torch)
        a8 = gemm_flops / (g8 / 1e3) / 1e12
        out["mxfp8_experts"] = {"value": round(T / (ms8 / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms8, 4),
                                "stage_ms": round(g8, 4), "achieved_tflops": round(a8, 1),
                                "peak_tflops": PEAK_FP8_TFLOPS, "frac": round(a8 / PEAK_FP8_TFLOPS, 4)}
        del layer8, w8
    if args.precision == "bf16" and not args.no_backward:
        # The routed experts' backward on the same routing (an extra record): input gradient of
        # the activation with the SwiGLU backward fused, w2's weight gradient, the input
        # gradient of z (scattered per copy, then summed per token) and w1's weight gradient.
        # Saved tensors from the training forward; output and workspace allocated outside the
        # timed region.
        fw = moe.experts_forward_train(cfg, w, z, offs, perm)
        dy = torch.randn(fw["y_assign"].shape, device="cuda").mul_(0.5).to(x.dtype)
        bws = torch.empty(moe.experts_backward_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
        grads = {"dz": torch.empty_like(z), "dw1": torch.empty_like(w["w1"]), "dw2": torch.empty_like(w["w2"])}
        run_bwd = lambda: moe.experts_backward(cfg, w, z, offs, perm, fw, dy, workspace=bws, out=grads)  # noqa: E731
        for _ in range(2):
            run_bwd()
        bms = event_time_ms(run_bwd, max(args.steps, 5), torch)
        ftms = event_time_ms(lambda: moe.experts_forward_train(cfg, w, z, offs, perm), max(args.steps, 5), torch)
        cbms = None
        if not (L and cfg.get("up_proj_input_norm", True)):  # no backward through the latent norm
            o_grad = torch.randn((T, K), device="cuda").to(x.dtype)
            cbms = event_time_ms(lambda: moe.combine_backward(cfg, fw["y_assign"], r["expert_weights"], o_grad), 5,
                                 torch)
        bflops = 12.0 * A * K * h
        ab = bflops / (bms / 1e3) / 1e12
        out["experts_backward"] = {"value": round(T / (bms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(bms, 4),
                                   "flops_per_launch": bflops, "achieved_tflops": round(ab, 1),
                                   "peak_tflops": PEAK_BF16_TFLOPS, "frac": round(ab / PEAK_BF16_TFLOPS, 4),
                                   "forward_train_ms": round(ftms, 4),
                                   "combine_backward_ms": None if cbms is None else round(cbms, 4)}
        del fw, dy, bws, grads
    if args.stages:
        st = {}
        st["router"] = event_time_ms(lambda: moe.router_forward(cfg, w, x, logits=False, scores=False), 5, torch)
        idx = moe.router_forward(cfg, w, x, logits=False, scores=False)["expert_indices"]
        st["permute"] = event_time_ms(lambda: moe.permute(cfg, idx), 5, torch)
        if L:
            st["latent_down"] = event_time_ms(lambda: moe.latent_down(cfg, w, x), 5, torch)
        st["experts"] = gemm_ms
        ya = moe.experts_forward(cfg, w, z, offs, perm)
        st["combine"] = event_time_ms(lambda: moe.combine(cfg, ya, r["expert_weights"], w.get("norm_weight")), 5,
                                      torch)
        if L:
            n = torch.empty((T, L), dtype=x.dtype, device=x.device)
            st["latent_up"] = event_time_ms(lambda: moe.latent_up(cfg, w, n), 5, torch)
        out["stages_ms"] = {k2: round(v, 4) for k2, v in st.items()}
    if not args.no_calibration:
        # Rates this device achieves (the published peaks assume clocks the chip does not hold
        # under sustained matrix load): the library's register-only matrix-core loop and its
        # 16-byte-vector copy, timed with HIP events on the current stream.
        cal = calibration(moe, torch)
        out["calibration"] = cal
        out["roofline"]["achievable_peak"] = cal["mfma_bf16_tflops"]
        out["roofline"]["frac_of_achievable"] = round(achieved / cal["mfma_bf16_tflops"], 4)
        if "mxfp8_experts" in out:
            mxr = out["mxfp8_experts"]
            mxr["achievable_peak_tflops"] = cal["mfma_mxfp8_tflops"]
            mxr["frac_of_achievable"] = round(mxr["achieved_tflops"] / cal["mfma_mxfp8_tflops"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, w, x, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
