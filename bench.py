#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer forward on one MI355X.

A step is one full forward of the layer (router -> gating/top-k -> dispatch -> [latent down]
-> grouped SwiGLU experts -> combine [-> norm -> latent up]) over one batch of synthetic
tokens, with inputs and weights resident in HBM. Headline workload: the largest layer that
fits one GPU, the skewed-load layer (32768 tokens, d_model 4096, 256 experts, top-8, hidden
2048, sigmoid gating with score_bias 2 ln(1/(e+1)), bf16, fp32 router). The other four
workloads (tiny fp32, OlmoE-shaped, 896-expert latent, decode) are reported as extra
records of the same line.

Printed: one JSON line with tokens/s for the whole layer (wall clock over the timed steps),
per-step HIP-event times (median, p10, p90; without and with a last-level-cache flush between
steps), the roofline of the dominant stage (the grouped expert GEMMs, timed with HIP events on
the stream they run on; bound by the matrix cores or by HBM, whichever the stage's arithmetic
intensity says), per-stage algorithmic bytes and GB/s, the achievable rates of this device,
and the CPU oracle timed on a bounded sample of the headline workload.
"""
import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA (MXFP8 experts)
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
# matrix-core flop per clock of the whole chip: the published bf16 peak at 2.4 GHz
BF16_FLOP_PER_CLOCK = PEAK_BF16_TFLOPS * 1e12 / 2.4e9
HEADLINE = "skewed"
EXTRAS = ("olmoe", "latent896", "decode", "tiny_f32")
FLUSH_BYTES = 512 << 20    # twice the 256 MiB last-level cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, help="headline workload")
    ap.add_argument("--extra", default=",".join(EXTRAS),
                    help="comma-separated workloads reported as extra records ('' for none)")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--precision", default="bf16", choices=("bf16", "mxfp8"),
                    help="precision of the expert matmuls (mxfp8: block-scaled E4M3 on the fp8 matrix cores)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mxfp8", action="store_true",
                    help="skip the extra measurement of the same layer with MXFP8 expert matmuls")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the extra measurement of the routed experts' backward")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the measurement of the achievable matrix-core and copy rates")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor BLAS (torch linear, hipBLASLt) on one expert's dense GEMM "
                         "shapes of the headline workload (context for the grouped GEMM's rate)")
    ap.add_argument("--profile-run", action="store_true",
                    help="only run --warmup + --steps layer forwards of --workload (for counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times): the reference the HBM "
                         "byte counters are scaled by")
    ap.add_argument("--restage-traffic", metavar="JSON",
                    help="no GPU: recompute the stage sums of a traffic record from its per-kernel entries "
                         "(with this file's stage classification) and write it to profiles/")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="no GPU: print, per kernel of a rocprofv3 --pmc output folder, the dispatches, the "
                         "mean duration and the mean of each counter (one JSON line per kernel)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="no GPU: write profiles/traffic_<workload>.json from four rocprofv3 --pmc output "
                         "folders (FETCH_SIZE and WRITE_SIZE of --profile-run, then of --copy-calibration 256)")
    return ap.parse_args()


# --------------------------------------------------------------------------- counter records

CSRC = os.path.join(ROOT, "top_routing_grouped_router_amd", "csrc")
# the sources each stage's kernels are built from: a counter record taken on other sources
# describes other kernels and is not used
STAGE_SOURCES = {
    "router": ("router.hip", "gemm_bf16.hip", "gemm_f32.hip", "common.hpp"),
    "dispatch": ("dispatch.hip", "common.hpp"),
    "latent": ("gemm_bf16.hip", "gemm_skinny.hip", "common.hpp"),
    "experts": ("gemm_bf16.hip", "gemm_f32.hip", "common.hpp"),
    "combine": ("combine.hip", "common.hpp"),
}


def _code_only(text):
    """The source with comments and blank space removed (string literals kept as written), so
    that a comment-only edit leaves the hash of the code unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch == '"' or ch == "'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def sources_sha256(names):
    """Hash of the code (comments and layout aside) of the sources a stage's kernels build from:
    a traffic record applies while it matches."""
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def _gemm_flags(name):
    """Template flags after the tile shape of a gemm_bf16_kernel name (SWIGLU, GATHER, SCATTER,
    then output / operand-layout / epilogue options)."""
    tail = name.split(">", 1)[1] if ">" in name else name
    return [t.strip() for t in tail.split(">")[0].split(",")][1:]


def kernel_stage(name):
    """Which stage of the forward a kernel of the layer belongs to."""
    if any(k in name for k in ("router_mfma_kernel", "split_planes_kernel", "gate_topk_kernel")):
        return "router"
    if any(k in name for k in ("rank_kernel", "scan_cols_kernel", "offsets_tiles_kernel", "permute_kernel",
                               "dispatch_small_kernel")):
        return "dispatch"
    if "combine" in name:
        return "combine"
    if "gemm_skinny" in name:
        return "latent"
    if "gemm_bf16_kernel" in name:
        # Shape<WM, WN, TM, TN, BK, NSTAGE, WG_PER_CU, PLANES, ...>: three weight planes = router
        shape = name.split("Shape<", 1)[1].split(">", 1)[0].split(",") if "Shape<" in name else []
        if "ShapeRouter" in name or (len(shape) > 7 and shape[7].strip() == "3"):
            return "router"
        f = _gemm_flags(name)
        if f[:3] == ["true", "true", "false"] or f[:3] == ["false", "false", "true"]:
            return "experts"
        return "latent"
    if "gemm_f32" in name:
        return "experts"  # the fp32 layer's router logits run on it too; it is one kernel name
    if "zero_dropped" in name:
        return "experts"
    return None


def _counter_rows(folder):
    """(kernel name, counter value) per dispatch from a rocprofv3 --pmc csv output folder."""
    import csv
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    with open(files[0]) as f:
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(f)]


def counter_summary(folder):
    """Per kernel of a rocprofv3 --pmc csv folder: dispatches, mean duration (ns) and the mean of
    each counter per dispatch; derived for the clock and matrix-core counters: the shader clock
    (GRBM_GUI_ACTIVE over the 8 XCDs / duration) and the matrix-core busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs / the active cycles of one XCD)."""
    import csv
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    agg = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            k = agg.setdefault(r["Kernel_Name"], {"dispatch": set(), "dur": {}, "ctr": {}})
            d = r.get("Dispatch_Id") or r.get("Correlation_Id")
            k["dispatch"].add(d)
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                k["dur"][d] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            k["ctr"].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    for name, k in agg.items():
        n = len(k["dispatch"])
        rec = {"kernel": name, "stage": kernel_stage(name), "dispatches": n,
               "mean_ns": round(sum(k["dur"].values()) / len(k["dur"]), 1) if k["dur"] else None}
        for cn, vals in k["ctr"].items():
            rec[cn] = sum(vals) / len(vals)
        if rec["mean_ns"] and "GRBM_GUI_ACTIVE" in rec:
            rec["clock_ghz"] = round(rec["GRBM_GUI_ACTIVE"] / 8 / rec["mean_ns"], 3)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in rec:
                rec["mfma_busy"] = round(rec["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (rec["GRBM_GUI_ACTIVE"] / 8), 4)
        print(json.dumps(rec))


def record_traffic(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, steps, copy_mib=256):
    """HBM bytes per layer step and per stage: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of
    every kernel of a --profile-run, each scaled by what the same counter reads for a plain
    device copy of copy_mib MiB. A kernel's bytes per step = its summed counter over the run /
    the layer steps of the run. Written with the hash of each stage's sources."""
    def by_kernel(folder):
        out = {}
        for name, v in _counter_rows(folder):
            ent = out.setdefault(name, [0.0, 0])
            ent[0] += v
            ent[1] += 1
        return out

    def copy_kib(folder):
        vals = sorted((v for name, v in _counter_rows(folder) if "copyBuffer" in name), reverse=True)
        if not vals:
            raise SystemExit("copy calibration: no copy kernel in the profile")
        return sum(vals[:3]) / len(vals[:3])

    copied = float(copy_mib << 10)
    cf, cw = copy_kib(copy_fetch_dir), copy_kib(copy_write_dir)
    fs, ws = copied / cf, copied / cw
    fetch, write = by_kernel(fetch_dir), by_kernel(write_dir)
    kernels = {}
    stages = {}
    for name in sorted(set(fetch) | set(write)):
        st = kernel_stage(name)
        if st is None:
            continue
        fb = fetch.get(name, [0.0, 1])
        wb = write.get(name, [0.0, 1])
        rec = {"stage": st, "dispatches_per_step": fb[1] / steps,
               "fetch_bytes_per_step": fb[0] * 1024 * fs / steps, "write_bytes_per_step": wb[0] * 1024 * ws / steps}
        kernels[name] = rec
        s = stages.setdefault(st, {"fetch_bytes": 0.0, "write_bytes": 0.0})
        s["fetch_bytes"] += rec["fetch_bytes_per_step"]
        s["write_bytes"] += rec["write_bytes_per_step"]
    for st, s in stages.items():
        s["bytes"] = int(round(s["fetch_bytes"] + s["write_bytes"]))
        s["source_sha256"] = sources_sha256(STAGE_SOURCES[st])
    rec = {
        "workload": workload,
        "what": "HBM bytes per layer step from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of "
                "`bench.py --workload W --profile-run`, scaled by the same counters' reading for a "
                "plain device copy (bench.py --copy-calibration 256)",
        "layer_steps_in_run": steps,
        "copy_calibration": {"bytes_copied_kib": copied, "fetch_size_kib": cf, "write_size_kib": cw,
                             "fetch_scale": fs, "write_scale": ws},
        "stages": stages,
        "kernels": kernels,
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"workload": workload, "stages": stages}))


def restage_traffic(path):
    """Stage sums of a traffic record from its per-kernel entries, classified by kernel_stage;
    the stage source hashes are kept from the record where the stage existed (they describe the
    sources the counters were taken on), else taken from the current sources."""
    with open(path) as f:
        rec = json.load(f)
    old = rec.get("stages", {})
    stages = {}
    for name, k in rec["kernels"].items():
        st = kernel_stage(name)
        k["stage"] = st
        if st is None:
            continue
        s = stages.setdefault(st, {"fetch_bytes": 0.0, "write_bytes": 0.0})
        s["fetch_bytes"] += k["fetch_bytes_per_step"]
        s["write_bytes"] += k["write_bytes_per_step"]
    for st, s in stages.items():
        s["bytes"] = int(round(s["fetch_bytes"] + s["write_bytes"]))
        s["source_sha256"] = old.get(st, {}).get("source_sha256") or sources_sha256(STAGE_SOURCES[st])
    rec["stages"] = stages
    out = os.path.join(ROOT, "profiles", f"traffic_{rec['workload']}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"workload": rec["workload"], "stages": stages}))


def recorded_stage_traffic(workload):
    """Stage -> HBM bytes per step from the committed counter record, for the stages whose
    kernel sources are unchanged since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return {}
    with open(p) as f:
        rec = json.load(f)
    out = {}
    for st, s in rec.get("stages", {}).items():
        if st in STAGE_SOURCES and s.get("source_sha256") == sources_sha256(STAGE_SOURCES[st]):
            out[st] = s["bytes"]
    return out


# --------------------------------------------------------------------------- timing

def event_times_ms(fn, n, torch, before=None):
    """GPU time of each of n calls of fn() on the current stream, each between its own pair of
    HIP events; `before` (if given) runs before each call, outside the events."""
    evs = []
    for _ in range(n):
        if before is not None:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def batch_time_ms(fn, n, torch):
    """Average GPU time of fn() over n back-to-back calls between one pair of events (the
    calls' host overhead overlaps the queued GPU work)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def pstats(ts):
    import numpy as np
    a = np.asarray(ts, np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4), "n": int(a.size)}


def sysfs_sclk_mhz():
    """Current shader clock of the first GPU whose DPM table sysfs exposes (the level marked
    '*'), or None."""
    for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(p) as f:
                for line in f:
                    if "*" in line:
                        return float(line.split(":")[1].strip().split("M")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


def calibration(moe, torch):
    """Achievable matrix-core rates (TFLOP/s: bf16, and the block-scaled FP8 of the MXFP8 experts)
    and HBM copy rate (GB/s of read + write) of this device, each the median of 5 event-timed
    launches of the library's calibration kernels (about 3 ms each)."""
    def loop_rate(run):
        out, _ = run(200)
        t = batch_time_ms(lambda: run(200, out), 3, torch)
        iters = max(200, int(200 * 3.0 / max(t, 1e-3)))
        run(iters, out)
        ts = sorted(event_times_ms(lambda: run(iters, out), 5, torch))
        return run(iters, out)[1] / (ts[2] / 1e3) / 1e12, iters, ts[2]

    bf16, iters, ms = loop_rate(moe.calibrate_mfma_bf16)
    mx, mx_iters, mx_ms = loop_rate(moe.calibrate_mfma_mxfp8)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    moe.calibrate_copy(src, dst)
    cs = sorted(event_times_ms(lambda: moe.calibrate_copy(src, dst), 5, torch))
    del src, dst
    return {"mfma_bf16_tflops": round(bf16, 1), "mfma_loop_iters": iters, "mfma_loop_ms": round(ms, 4),
            "mfma_loop_effective_clock_mhz": round(bf16 * 1e12 / BF16_FLOP_PER_CLOCK / 1e6, 0),
            "mfma_mxfp8_tflops": round(mx, 1), "mfma_mxfp8_loop_iters": mx_iters,
            "mfma_mxfp8_loop_ms": round(mx_ms, 4),
            "copy_gbs": round(2 * nbytes / (cs[2] / 1e3) / 1e9, 1), "copy_bytes": nbytes,
            "copy_ms": round(cs[2], 4)}


# --------------------------------------------------------------------------- work models

def work_model(cfg, T, n_touched):
    """Algorithmic flops and HBM bytes of each stage of one forward (what the computation must
    read and write, not what the kernels do): the router reads x and the fp32 router weights
    and writes indices and weights; the dispatch reads the indices and writes counts, offsets,
    permutation and inverse; the experts read the weights of the experts that received tokens,
    each token's z row once, write and read the SwiGLU activation and write Y; the combine reads
    Y and the weights and writes one row per token; the latent projections read their input and
    weight and write their output."""
    es = 2 if cfg["dtype"] == "bf16" else 4
    E, k, h, d = cfg["num_experts"], cfg["top_k"], cfg["hidden_size"], cfg["d_model"]
    L = cfg["latent_dim"] or 0
    K = L or d
    A = T * k
    m = {
        "router": {"flops": 2.0 * T * d * E, "bytes": T * d * es + E * d * 4 + A * 8},
        "dispatch": {"flops": 0.0, "bytes": A * 4 + A * 8 + (2 * E + 1) * 4},
        "experts": {"flops": 6.0 * A * K * h,
                    "bytes": 3 * K * h * es * n_touched + T * K * es + 2 * A * h * es + A * K * es},
        "combine": {"flops": 2.0 * A * K, "bytes": A * K * es + A * 4 + T * K * es + (L * 4 if L else 0)},
    }
    if L:
        m["latent_down"] = {"flops": 2.0 * T * d * L, "bytes": T * d * es + L * d * es + T * L * es}
        m["latent_up"] = {"flops": 2.0 * T * L * d, "bytes": T * L * es + d * L * es + T * d * es}
    return m


def bound_of(cfg, flops, nbytes):
    """The roof a stage sits under: the matrix cores when its arithmetic intensity is above the
    ridge point (peak flop/s over HBM bytes/s), else HBM; fp32 layers run on the fp32 vector
    ALUs."""
    if cfg["dtype"] == "f32":
        return ("alu", PEAK_F32_TFLOPS) if flops / max(nbytes, 1) > PEAK_F32_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) \
            else ("hbm", PEAK_HBM_GBS)
    return ("mfma", PEAK_BF16_TFLOPS) if flops / max(nbytes, 1) > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) \
        else ("hbm", PEAK_HBM_GBS)


class StageRunner:
    """Each stage of the forward enqueued alone through the C ABI on preallocated buffers (the
    binding's marshalling only), so that a batch of calls can be timed between two events."""

    def __init__(self, moe, torch, cfg, w, x, layer):
        self.moe, self.torch = moe, torch
        c = moe.MoEConfig.of(cfg)
        self.c, self.cw = c.to_c(), moe._c_weights(c, w)
        T, E, k = x.shape[0], c.num_experts, c.top_k
        self.T, self.K, self.L = T, c.expert_dim, c.latent_dim or 0
        dev = x.device
        self.r = moe._routing_tensors(c, T, dev, moe.ROUTING_FIELDS)
        self.ws = layer.workspace(T, dev)
        self.x = x
        self.z = torch.empty((T, self.L), dtype=x.dtype, device=dev) if self.L else x
        self.ya = torch.empty((T * k, self.K), dtype=x.dtype, device=dev)
        self.o = torch.empty((T, self.K), dtype=x.dtype, device=dev)
        self.y = torch.empty_like(x)
        self.cr = moe._c_routing({n: self.r[n] for n in ("expert_weights", "expert_indices")})
        self.s = moe._stream()
        P = moe._ptr
        self.p = {n: P(t) for n, t in self.r.items()}
        self.px, self.pz, self.pya, self.po, self.py, self.pws = P(x), P(self.z), P(self.ya), P(self.o), P(self.y), \
            P(self.ws)
        self.nws = self.ws.numel()
        # fill the routing once with the whole layer
        layer(x, out=self.y, routing=None)
        self.router()
        self.permute()
        if self.L:
            self.latent_down()
        torch.cuda.synchronize()

    def router(self):
        m = self.moe
        m._check(m._router_forward(ctypes.byref(self.c), ctypes.byref(self.cw), self.T, self.px, ctypes.byref(self.cr),
                                   self.pws, self.nws, self.s))

    def permute(self):
        m, p = self.moe, self.p
        m._check(m._permute(ctypes.byref(self.c), self.T, p["expert_indices"], p["batch_size_per_expert"],
                            p["expert_offsets"], p["permutation"], p["inverse_permutation"], self.pws, self.nws,
                            self.s))

    def latent_down(self):
        m = self.moe
        m._check(m._latent_down(ctypes.byref(self.c), ctypes.byref(self.cw), self.T, self.px, self.pz, self.pws,
                                self.nws, self.s))

    def experts(self):
        m, p = self.moe, self.p
        m._check(m._experts_forward(ctypes.byref(self.c), ctypes.byref(self.cw), self.T, self.pz, p["expert_offsets"],
                                    p["permutation"], self.pya, self.pws, self.nws, self.s))

    def combine(self):
        m, p = self.moe, self.p
        m._check(m._combine(ctypes.byref(self.c), ctypes.byref(self.cw), self.T, self.pya, p["expert_weights"],
                            self.po, self.s))

    def latent_up(self):
        m = self.moe
        m._check(m._latent_up(ctypes.byref(self.c), ctypes.byref(self.cw), self.T, self.po, self.py, self.pws,
                              self.nws, self.s))


def measure_layer(moe, torch, name, cfg, w, x, steps, warmup, flush_buf, precision="bf16"):
    """Wall-clock tokens/s over `steps` back-to-back forwards, per-step event times with and
    without a cache flush between steps, per-stage times, algorithmic work and the roofline of
    the expert stage."""
    T = x.shape[0]
    layer = moe.MoELayer(dict(cfg, expert_precision=precision), w)
    y = torch.empty_like(x)
    for _ in range(warmup):
        layer(x, out=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer(x, out=y)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    sclk = sysfs_sclk_mhz()
    ev = event_times_ms(lambda: layer(x, out=y), steps, torch)
    flushed = event_times_ms(lambda: layer(x, out=y), steps, torch, before=lambda: flush_buf.fill_(1))

    run = StageRunner(moe, torch, dict(cfg, expert_precision=precision), layer.weights, x, layer)
    counts = run.r["batch_size_per_expert"].cpu()
    n_touched = int((counts > 0).sum())
    model = work_model(cfg, T, n_touched)
    reps = max(steps, 5)
    stage_ms = {"router": batch_time_ms(run.router, reps, torch), "dispatch": batch_time_ms(run.permute, reps, torch)}
    if run.L:
        stage_ms["latent_down"] = batch_time_ms(run.latent_down, reps, torch)
    stage_ms["experts"] = pstats(event_times_ms(run.experts, reps, torch))["mean"]
    stage_ms["combine"] = batch_time_ms(run.combine, reps, torch)
    if run.L:
        stage_ms["latent_up"] = batch_time_ms(run.latent_up, reps, torch)
    traffic = recorded_stage_traffic(name) if precision == "bf16" else {}
    stages = {}
    for st, t in stage_ms.items():
        mdl = model[st]
        rec = {"ms": round(t, 4), "bytes": int(mdl["bytes"]), "gbs": round(mdl["bytes"] / (t / 1e3) / 1e9, 1),
               "hbm_frac": round(mdl["bytes"] / (t / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
        if mdl["flops"]:
            rec["flops"] = mdl["flops"]
            rec["tflops"] = round(mdl["flops"] / (t / 1e3) / 1e12, 2)
        tk = {"latent_down": "latent", "latent_up": "latent"}.get(st, st)
        if tk in traffic and tk == st:
            rec["traffic_bytes"] = traffic[tk]
        stages[st] = rec

    ex = model["experts"]
    gemm_ms = stage_ms["experts"]
    bound, peak = bound_of(cfg, ex["flops"], ex["bytes"])
    if precision == "mxfp8":
        bound, peak = "mfma", PEAK_FP8_TFLOPS
    if bound in ("mfma", "alu"):
        achieved, unit = ex["flops"] / (gemm_ms / 1e3) / 1e12, "TFLOP/s"
    else:
        achieved, unit = ex["bytes"] / (gemm_ms / 1e3) / 1e9, "GB/s"
    E, d, L = cfg["num_experts"], cfg["d_model"], cfg["latent_dim"] or 0
    layer_flops = sum(v["flops"] for v in model.values())
    out = {
        "value": round(T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms, 4),
        "step_ms_events": pstats(ev),
        "step_ms_events_cache_flushed": pstats(flushed),
        "layer_tflops": round(layer_flops / (ms / 1e3) / 1e12, 2),
        "experts_touched": n_touched,
        "max_over_mean_load": round(float(counts.max()) / max(float(counts.float().mean()), 1e-30), 2),
        "roofline": {"kernel": "grouped expert GEMMs (up/gate + SwiGLU, down): one moe_experts_forward call",
                     "bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic.get("experts"),
                     "stage_ms": round(gemm_ms, 4), "flops_per_launch": ex["flops"], "bytes_per_launch": ex["bytes"],
                     "intensity_flop_per_byte": round(ex["flops"] / ex["bytes"], 1)},
        "stages": stages,
        "sysfs_sclk_mhz_after_steps": sclk,
    }
    del run, layer
    return out


def vendor_dense_gemm(cfg, w, rows, torch, reps=10):
    """The vendor BLAS (torch.nn.functional.linear on bf16: hipBLASLt) on the dense shapes of
    the busiest expert: M = its rows, GEMM1 (M, K) x (2h, K)^T and GEMM2 (M, h) x (K, h)^T, on
    random rows. Context for the grouped kernels' rate (which also gather, scatter and fuse
    SwiGLU); not part of the layer."""
    import torch.nn.functional as F
    h = cfg["hidden_size"]
    K = cfg["latent_dim"] or cfg["d_model"]
    e = int(torch.argmax(rows))
    M = int(rows[e])
    g = torch.Generator(device="cuda").manual_seed(0)
    a1 = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    a2 = torch.randn((M, h), generator=g, device="cuda").to(torch.bfloat16)
    w1, w2 = w["w1"][e].contiguous(), w["w2"][e].contiguous()
    for _ in range(2):
        F.linear(a1, w1)
        F.linear(a2, w2)
    t1 = pstats(event_times_ms(lambda: F.linear(a1, w1), reps, torch))["median"]
    t2 = pstats(event_times_ms(lambda: F.linear(a2, w2), reps, torch))["median"]
    f1, f2 = 2.0 * M * 2 * h * K, 2.0 * M * K * h
    return {"what": "torch.nn.functional.linear (hipBLASLt), bf16, the busiest expert's dense shapes",
            "rows": M, "gemm1_ms": round(t1, 4), "gemm1_tflops": round(f1 / (t1 / 1e3) / 1e12, 1),
            "gemm2_ms": round(t2, 4), "gemm2_tflops": round(f2 / (t2 / 1e3) / 1e12, 1),
            "pair_tflops": round((f1 + f2) / ((t1 + t2) / 1e3) / 1e12, 1)}


# --------------------------------------------------------------------------- CPU baseline

def host_description():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    threads = None
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')} ({info[0].get('architecture')})"
            threads = max(p.get("num_threads", 1) for p in info)
    except Exception:  # pragma: no cover
        pass
    return model, blas, threads


def cpu_baseline(cfg, w, x, target_s):
    """The oracle (float32-accumulation mode, plain NumPy) timed on the first n tokens of the
    batch: n is chosen from a 128-token pilot so that the timed run takes about target_s. Only
    the experts those tokens route to are copied to the host (the oracle computes only experts
    that received tokens). The layer is token-independent, so tokens/s on the sample is the
    whole batch's rate."""
    import numpy as np
    import workloads
    from oracle import moe_oracle as O
    cfgO = O.MoEConfig.from_dict(cfg)
    T = x.shape[0]
    small = {k: workloads.to_numpy_f32(v) for k, v in w.items() if k not in ("w1", "w2")}

    def weights_for(xs):
        l = O.router_logits(xs, small["router_weight"], small["router_bias"], acc=np.float32)
        idx = O.route(cfgO, l, small["score_bias"])["idx"]
        used = np.unique(idx)
        return dict(small, w1={int(e): workloads.to_numpy_f32(w["w1"][int(e)]) for e in used},
                    w2={int(e): workloads.to_numpy_f32(w["w2"][int(e)]) for e in used}), len(used)

    def timed(n):
        xs = workloads.to_numpy_f32(x[:n])
        wo, used = weights_for(xs)
        t0 = time.perf_counter()
        O.forward(cfgO, wo, xs, acc=np.float32)
        return time.perf_counter() - t0, used

    n0 = min(128, T)
    t_pilot, _ = timed(n0)
    n = int(min(T, max(n0, n0 * target_s / max(t_pilot, 1e-6))))
    n = max(n0, n // n0 * n0) if n < T else T
    dt, used = timed(n)
    model, blas, threads = host_description()
    return {"value": round(n / dt, 1), "unit": "tokens/s", "cores": int(threads or os.cpu_count() or 1),
            "kind": "oracle",
            "sample": f"first {n} of the {T} tokens (oracle in float32-accumulation mode; the {used} experts "
                      f"those tokens use; {dt:.1f} s)",
            "cpu_model": model, "blas": blas, "host_threads_available": len(os.sched_getaffinity(0))}


# --------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic, steps=args.warmup + args.steps)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.restage_traffic:
        restage_traffic(args.restage_traffic)
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
    cfg, w, x = workloads.make_workload(name, device="cuda")
    if args.profile_run:
        layer = moe.MoELayer(dict(cfg, expert_precision=args.precision), w)
        y = torch.empty_like(x)
        for _ in range(args.warmup + args.steps):
            layer(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": name, "layer_steps": args.warmup + args.steps}), flush=True)
        return

    T = x.shape[0]
    E, k, h = cfg["num_experts"], cfg["top_k"], cfg["hidden_size"]
    d, L = cfg["d_model"], cfg["latent_dim"] or 0
    K = L or d
    A = T * k
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    head = measure_layer(moe, torch, name, cfg, w, x, args.steps, args.warmup, flush_buf, args.precision)

    out = {
        "metric": "MoE layer fwd tokens/s + grouped-GEMM % of bf16 MFMA peak, 1xMI355X",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp8 experts, bf16" if args.precision == "mxfp8" else "bf16") if cfg["dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": name, "tokens": T, "d_model": d, "num_experts": E, "top_k": k,
                   "hidden_size": h, "latent_dim": L or None, "gating": cfg["gating_function"],
                   "router": "fp32", "expert_precision": args.precision, "parallelism": "none (1 GPU)"},
        "timing": "value = tokens / (wall clock of `steps` back-to-back forwards / steps), bracketed by "
                  "device synchronisation, the last-level cache not flushed; step_ms_events: each step between "
                  "HIP events; step_ms_events_cache_flushed: the same with a 512 MiB write between steps",
    }
    out.update({k2: v for k2, v in head.items() if k2 not in ("value", "unit", "ms_per_step")})
    gemm_flops = 6.0 * A * K * h

    if args.precision == "bf16" and cfg["dtype"] == "bf16" and not args.no_mxfp8:
        # The same layer with the expert matmuls in MXFP8 (block-scaled E4M3; weights quantised
        # once, outside the timed region): an extra record, not the headline.
        mx = measure_layer(moe, torch, name, cfg, moe.quantize_expert_weights(w), x, args.steps, args.warmup,
                           flush_buf, "mxfp8")
        g8 = mx["roofline"]["stage_ms"]
        a8 = gemm_flops / (g8 / 1e3) / 1e12
        out["mxfp8_experts"] = {"value": mx["value"], "unit": "tokens/s", "ms_per_step": mx["ms_per_step"],
                                "step_ms_events": mx["step_ms_events"], "stage_ms": g8,
                                "achieved_tflops": round(a8, 1), "peak_tflops": PEAK_FP8_TFLOPS,
                                "frac": round(a8 / PEAK_FP8_TFLOPS, 4)}
        del mx
        torch.cuda.empty_cache()
    if args.precision == "bf16" and not args.no_backward:
        # The routed experts' backward on the same routing (an extra record): input gradient of
        # the activation with the SwiGLU backward fused, w2's weight gradient, the input
        # gradient of z (scattered per copy, then summed per token) and w1's weight gradient.
        # Saved tensors from the training forward; output and workspace allocated outside the
        # timed region.
        layer = moe.MoELayer(cfg, w)
        _, r = layer(x, routing=("expert_offsets", "permutation", "expert_weights"))
        z = moe.latent_down(cfg, w, x) if L else x
        offs, perm = r["expert_offsets"], r["permutation"]
        fw = moe.experts_forward_train(cfg, w, z, offs, perm)
        dy = torch.randn(fw["y_assign"].shape, device="cuda").mul_(0.5).to(x.dtype)
        bws = torch.empty(moe.experts_backward_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
        grads = {"dz": torch.empty_like(z), "dw1": torch.empty_like(w["w1"]), "dw2": torch.empty_like(w["w2"])}
        run_bwd = lambda: moe.experts_backward(cfg, w, z, offs, perm, fw, dy, workspace=bws, out=grads)  # noqa: E731
        for _ in range(2):
            run_bwd()
        bms = pstats(event_times_ms(run_bwd, max(args.steps, 5), torch))["mean"]
        ftms = pstats(event_times_ms(lambda: moe.experts_forward_train(cfg, w, z, offs, perm), max(args.steps, 5),
                                     torch))["mean"]
        cbms = None
        if not (L and cfg.get("up_proj_input_norm", True)):  # no backward through the latent norm
            o_grad = torch.randn((T, K), device="cuda").to(x.dtype)
            cbms = pstats(event_times_ms(lambda: moe.combine_backward(cfg, fw["y_assign"], r["expert_weights"],
                                                                      o_grad), 5, torch))["mean"]
        bflops = 12.0 * A * K * h
        ab = bflops / (bms / 1e3) / 1e12
        out["experts_backward"] = {"value": round(T / (bms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(bms, 4),
                                   "flops_per_launch": bflops, "achieved_tflops": round(ab, 1),
                                   "peak_tflops": PEAK_BF16_TFLOPS, "frac": round(ab / PEAK_BF16_TFLOPS, 4),
                                   "forward_train_ms": round(ftms, 4),
                                   "combine_backward_ms": None if cbms is None else round(cbms, 4)}
        del fw, dy, bws, grads, layer, z, r
        torch.cuda.empty_cache()
    if not args.no_calibration:
        # Rates this device achieves (the published peaks assume clocks the chip does not hold
        # under sustained matrix load): the library's register-only matrix-core loop and its
        # 16-byte-vector copy, timed with HIP events on the current stream.
        cal = calibration(moe, torch)
        out["calibration"] = cal
        rf = out["roofline"]
        if rf["unit"] == "TFLOP/s" and cfg["dtype"] == "bf16":
            rf["achievable_peak"] = cal["mfma_bf16_tflops"] if args.precision == "bf16" else cal["mfma_mxfp8_tflops"]
        elif rf["unit"] == "GB/s":
            rf["achievable_peak"] = cal["copy_gbs"]
        if "achievable_peak" in rf:
            rf["frac_of_achievable"] = round(rf["achieved"] / rf["achievable_peak"], 4)
        if "mxfp8_experts" in out:
            mxr = out["mxfp8_experts"]
            mxr["achievable_peak_tflops"] = cal["mfma_mxfp8_tflops"]
            mxr["frac_of_achievable"] = round(mxr["achieved_tflops"] / cal["mfma_mxfp8_tflops"], 4)
    if args.vendor_gemm and cfg["dtype"] == "bf16":
        layer = moe.MoELayer(cfg, w)
        _, r = layer(x, routing=("batch_size_per_expert",))
        out["vendor_dense_gemm"] = vendor_dense_gemm(cfg, w, r["batch_size_per_expert"], torch)
        del layer, r
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, w, x, args.cpu_seconds)
    del w, x
    torch.cuda.empty_cache()

    extras = [] if args.no_extra else [e for e in args.extra.split(",") if e and e != name]
    if extras:
        out["workloads"] = {}
    for en in extras:
        ecfg, ew, ex = workloads.make_workload(en, device="cuda")
        rec = measure_layer(moe, torch, en, ecfg, ew, ex, args.steps, args.warmup, flush_buf)
        rec["config"] = {"tokens": ex.shape[0], "d_model": ecfg["d_model"], "num_experts": ecfg["num_experts"],
                         "top_k": ecfg["top_k"], "hidden_size": ecfg["hidden_size"],
                         "latent_dim": ecfg["latent_dim"], "gating": ecfg["gating_function"], "dtype": ecfg["dtype"]}
        if "calibration" in out:
            rf = rec["roofline"]
            if rf["unit"] == "GB/s":
                rf["achievable_peak"] = out["calibration"]["copy_gbs"]
            elif ecfg["dtype"] == "bf16":
                rf["achievable_peak"] = out["calibration"]["mfma_bf16_tflops"]
            if "achievable_peak" in rf:
                rf["frac_of_achievable"] = round(rf["achieved"] / rf["achievable_peak"], 4)
        out["workloads"][en] = rec
        del ew, ex
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
