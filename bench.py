"""Benchmark of the DeepSeekMoE layer forward pass on one MI355X.

One step = one call of moe_layer_forward (router, dispatch, routed + shared expert FFNs,
combine + residual) over the V3-style workload: T=16384 tokens, H=7168, 1 shared + 256 routed
SwiGLU experts of width 2048, top-8, sigmoid + selection bias, bf16 with fp32 accumulation.
Inputs are seeded synthetic tensors of that shape (no trained weights), resident in HBM before
timing starts.  The routed expert banks and the shared experts' gate/up bank are stored in fragment
order by default (moe_pack_weights, done once when the weights are loaded, outside the timed steps;
--weights unpacked keeps the [out, in] layout, with bit-identical results).  The decode regime (the first 128 tokens of the
same inputs) is timed as well.

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

METRIC = "MoE-layer tokens/s and TFLOP/s (% bf16 MFMA peak) at V3-style shape; decode HBM GB/s"
# routed gate/up grouped GEMM + SwiGLU: [out, in] banks, and banks in fragment order (moe_pack_weights)
DOMINANT_KERNELS = ("k_gemm_bf16_w4<0, true>", "k_gemm_bf16_w4p<0, false, 4, true>")


def dominant_kernel(flags):
    return DOMINANT_KERNELS[1] if flags else DOMINANT_KERNELS[0]

KERNEL_SOURCES = ["fine_grained_shared_amd/csrc/ffn.hip", "fine_grained_shared_amd/csrc/kernels.hpp",
                  "fine_grained_shared_amd/csrc/common.hpp"]
TRAFFIC_FILE = "profiles/traffic_ffn_up_v3_prefill.json"
COPY_BYTES = 1 << 30
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


# ---------------------------------------------------------------- algorithmic work counters

def ffn_params(n_experts, H, I, act_swiglu=True):
    """Weights of n_experts FFNs of width I: SwiGLU has gate, up and down (3 H*I), ReLU two (2 H*I)."""
    return n_experts * (3 if act_swiglu else 2) * H * I


def ffn_flops_per_token(k, H, I, act_swiglu=True):
    """FLOPs (2 per multiply-add) of k expert FFNs of width I on one token."""
    return 2 * k * (3 if act_swiglu else 2) * H * I


def layer_flops(w, T=None):
    """Router GEMM plus the FFNs of the selected and shared experts (no padding, no elementwise)."""
    T = w.T if T is None else T
    sw = w.act == 1
    return 2 * T * w.H * w.N_r + T * ffn_flops_per_token(w.K_r + w.Ks, w.H, w.I, sw)


def routed_up_flops(w, T=None):
    """FLOPs of the routed gate/up GEMM (the dominant kernel): T*K_r rows x (2I or I) x H."""
    T = w.T if T is None else T
    n1 = 2 * w.I if w.act == 1 else w.I
    return 2 * T * w.K_r * n1 * w.H


def decode_bytes(w, n_touched, T=None):
    """HBM bytes a decode step must move at least: weights of the touched routed experts and of the
    shared experts, the centroids, the tokens in and the outputs out (bf16)."""
    T = w.T if T is None else T
    e = 2 if w.dtype == 1 else 4
    per_expert = ffn_params(1, w.H, w.I, w.act == 1) * e
    return n_touched * per_expert + w.Ks * per_expert + w.N_r * w.H * e + 2 * T * w.H * e


# ---------------------------------------------------------------- HBM traffic from rocprofv3 counters

def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of the dominant kernel from the committed counter summary, or None
    when the kernel sources changed since the counters were taken or they cover another kernel."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha256") != kernel_source_hash() or t.get("dominant_kernel") != kernel:
        return None
    return t.get("traffic_bytes_per_launch")


def _read_counters(d):
    """{kernel name: {counter: [per-dispatch values]}} from a rocprofv3 --pmc output directory."""
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                key = (r.get("Dispatch_Id"), r["Counter_Name"])
                out.setdefault(name, {}).setdefault(r["Counter_Name"], {}).setdefault(key, 0.0)
                out[name][r["Counter_Name"]][key] += float(r["Counter_Value"])
    return {k: {c: list(v.values()) for c, v in d2.items()} for k, d2 in out.items()}


def _short(name):
    n = name.split("(")[0]
    return n.replace("void ", "").replace("moe::", "")


def rocprof_summary(trace_dir, fetch_dir=None, write_dir=None, out_json=None, dom_name=DOMINANT_KERNELS[1]):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run (and optional FETCH_SIZE /
    WRITE_SIZE passes) for the profiles/ folder; dom_name is the dominant kernel of the profiled run."""
    lines = []
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    dom = None
    for f in stats:
        with open(f) as fh:
            rows = list(csv.DictReader(fh))
        lines.append("| kernel | calls | avg ms | total ms | % |")
        lines.append("|---|---|---|---|---|")
        for r in rows:
            nm = _short(r["Name"])
            avg = float(r["AverageNs"]) / 1e6
            lines.append("| %s | %s | %.4f | %.3f | %.1f |" % (nm, r["Calls"], avg, float(r["TotalDurationNs"]) / 1e6,
                                                              float(r["Percentage"])))
            if nm.endswith(dom_name):
                dom = avg
    res = {"dominant_kernel": dom_name, "avg_ms": dom}
    if fetch_dir and write_dir:
        fc, wc = _read_counters(fetch_dir), _read_counters(write_dir)

        def pick(cnt, pat, counter):
            vals = [v for k, d in cnt.items() if pat in _short(k) for v in d.get(counter, [])]
            return sum(vals) / len(vals) if vals else None

        def copy_ref(cnt, counter):
            # the 1 GiB device-to-device copy the bench issues before timing: the largest
            # runtime copy-kernel dispatch
            vals = [v for k, d in cnt.items() if "copyBuffer" in k for v in d.get(counter, [])]
            return max(vals) if vals else None
        copy_f = copy_ref(fc, "FETCH_SIZE")
        copy_w = copy_ref(wc, "WRITE_SIZE")
        k_f = pick(fc, dom_name, "FETCH_SIZE")
        k_w = pick(wc, dom_name, "WRITE_SIZE")
        if None not in (copy_f, copy_w, k_f, k_w):
            sf, sw = COPY_BYTES / (copy_f * 1024), COPY_BYTES / (copy_w * 1024)
            res.update({"copy_fetch_kib": copy_f, "copy_write_kib": copy_w, "fetch_kib_per_launch": k_f,
                        "write_kib_per_launch": k_w, "fetch_scale": sf, "write_scale": sw,
                        "traffic_bytes_per_launch": k_f * 1024 * sf + k_w * 1024 * sw,
                        "source_sha256": kernel_source_hash()})
            lines.append("")
            lines.append("HBM traffic of %s per launch: FETCH_SIZE %.0f KiB x %.3f + WRITE_SIZE %.0f KiB x %.3f "
                         "= %.3f GB (scales: a plain %d-byte device copy reads FETCH %.0f KiB / WRITE %.0f KiB)" % (
                             dom_name, k_f, sf, k_w, sw, res["traffic_bytes_per_launch"] / 1e9, COPY_BYTES,
                             copy_f, copy_w))
    if out_json:
        with open(out_json, "w") as fh:
            json.dump(res, fh, indent=1)
    return "\n".join(lines), res


def _csv_rows(d, pattern):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _dispatch_counters(d):
    """{dispatch id: (kernel name, {counter: value summed over the dispatch's rows})} of a --pmc run."""
    out = {}
    for r in _csv_rows(d, "*counter_collection.csv"):
        did = r.get("Dispatch_Id") or r.get("Correlation_Id")
        name, vals = out.setdefault(did, (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _dispatch_ns(d):
    """{dispatch id: duration in ns} from the kernel trace written by the same rocprofv3 run."""
    out = {}
    for r in _csv_rows(d, "*kernel_trace.csv"):
        did = r.get("Dispatch_Id") or r.get("Correlation_Id")
        out[did] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def _simd_count(d, default=1024):
    for r in _csv_rows(d, "*agent_info.csv"):
        for k in ("Simd_Count", "SIMD_Count", "simd_count"):
            if r.get(k) and r.get("Agent_Type", r.get("Type", "GPU")).upper().endswith("GPU") and float(r[k]) > 0:
                n = float(r[k])
                cus = float(r.get("Cu_Count") or r.get("Compute_Unit_Count") or 0)
                return int(n * cus) if 0 < n <= 8 and cus > 0 else int(n)
    return default


def counter_summary(pmc_dir, fetch_dir=None, write_dir=None, copy_bytes=COPY_BYTES, rdreq_dir=None):
    """Per-kernel table of a rocprofv3 run with --pmc SQ_VALU_MFMA_BUSY_CYCLES MfmaUtil GRBM_GUI_ACTIVE
    SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES --kernel-trace, plus optional FETCH_SIZE and WRITE_SIZE runs.

    MFMA busy % is rocprofv3's MfmaUtil: sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES / (max over XCDs of
    GRBM_GUI_ACTIVE x SIMDs).  The shader clock is that max GRBM_GUI_ACTIVE (recovered from the two) over
    the dispatch's duration.  Executed bf16 MFMA work is SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP.
    HBM bytes are FETCH_SIZE and WRITE_SIZE scaled by what they read for the bench's plain 1 GiB device
    copy (the largest copy-kernel dispatch of the run)."""
    disp = _dispatch_counters(pmc_dir)
    dur = _dispatch_ns(pmc_dir)
    simds = _simd_count(pmc_dir)
    per = {}
    for did, (name, v) in disp.items():
        if did not in dur or dur[did] <= 0:
            continue
        a = per.setdefault(_short(name), {"n": 0, "ns": 0.0, "util": 0.0, "clk": 0.0, "mops": 0.0, "clk_n": 0})
        a["n"] += 1
        a["ns"] += dur[did]
        util = v.get("MfmaUtil")
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES")
        if util is not None:
            a["util"] += util
        if util and busy:
            grbm_max = busy / (util / 100.0 * simds)
            a["clk"] += grbm_max / dur[did]
            a["clk_n"] += 1
        a["mops"] += v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
    traffic = {}
    if fetch_dir and write_dir:
        fc, wc = _read_counters(fetch_dir), _read_counters(write_dir)
        copy_f = max([x for k, d in fc.items() if "copyBuffer" in k for x in d.get("FETCH_SIZE", [])] or [0])
        copy_w = max([x for k, d in wc.items() if "copyBuffer" in k for x in d.get("WRITE_SIZE", [])] or [0])
        if copy_f > 0 and copy_w > 0:
            sf, sw = copy_bytes / (copy_f * 1024), copy_bytes / (copy_w * 1024)
            for k in set(fc) | set(wc):
                f = fc.get(k, {}).get("FETCH_SIZE", [])
                w = wc.get(k, {}).get("WRITE_SIZE", [])
                if f and w:
                    traffic[_short(k)] = (sum(f) / len(f) * 1024 * sf, sum(w) / len(w) * 1024 * sw)
            traffic["_scales"] = (sf, sw, copy_f, copy_w)
    rdreq = {}
    if rdreq_dir:
        # bytes of the L2-to-fabric read requests by size: 128 x RDREQ_128B + 64 x RDREQ_64B + 32 x RDREQ_32B
        rc = _read_counters(rdreq_dir)
        for k, d in rc.items():
            n = len(d.get("TCC_EA0_RDREQ_128B_sum", []))
            if n:
                b = (128 * sum(d["TCC_EA0_RDREQ_128B_sum"]) + 64 * sum(d.get("TCC_EA0_RDREQ_64B_sum", [0])) +
                     32 * sum(d.get("TCC_EA0_RDREQ_32B_sum", [0])))
                rdreq[_short(k)] = b / n
    lines = ["| kernel | dispatches | avg ms | MFMA busy % | shader clock GHz | executed bf16 TFLOP/s |"
             " read GB | written GB | HBM TB/s |" + (" read GB (requests) |" if rdreq else ""),
             "|---|---|---|---|---|---|---|---|---|" + ("---|" if rdreq else "")]
    res = {}
    for k in sorted(per, key=lambda k: -per[k]["ns"]):
        a = per[k]
        n = a["n"]
        ms = a["ns"] / n / 1e6
        util = a["util"] / n
        # the counters cover the dispatch plus the profiler's own set-up around it, so the clock is
        # only meaningful for dispatches far longer than that (here: 0.5 ms and more)
        clk = a["clk"] / a["clk_n"] if a["clk_n"] and ms >= 0.5 else float("nan")
        tfs = a["mops"] / n * 512 / (ms * 1e-3) / 1e12
        rd = wr = tbs = None
        if k in traffic:
            rd, wr = traffic[k]
            tbs = (rd + wr) / (ms * 1e-3) / 1e12
        res[k] = {"dispatches": n, "avg_ms": ms, "mfma_busy_pct": util, "clock_ghz": clk,
                  "executed_tflops": tfs, "read_bytes": rd, "write_bytes": wr}
        lines.append("| %s | %d | %.4f | %.1f | %s | %.0f | %s | %s | %s |" % (
            k, n, ms, util, "-" if clk != clk else "%.2f" % clk, tfs, "-" if rd is None else "%.3f" % (rd / 1e9),
            "-" if wr is None else "%.3f" % (wr / 1e9), "-" if tbs is None else "%.2f" % tbs) +
            ((" %s |" % ("-" if k not in rdreq else "%.3f" % (rdreq[k] / 1e9))) if rdreq else ""))
    if "_scales" in traffic:
        sf, sw, cf, cw = traffic["_scales"]
        lines.append("")
        lines.append("Byte scales from the %d-byte device copy: FETCH_SIZE %.0f KiB -> x %.3f, WRITE_SIZE %.0f KiB "
                     "-> x %.3f.  SIMDs: %d." % (copy_bytes, cf, sf, cw, sw, simds))
    return "\n".join(lines), res


def power_summary(log, busy_mhz=1000.0):
    """Socket power and shader clocks from a log of `amd-smi metric --power --clock --json` samples, each
    preceded by a line `t=<unix seconds> phase=<label>` (the label names what the GPU was running):
    medians per phase over the samples with the clocks above busy_mhz (the GPU working)."""
    import re
    import statistics
    with open(log) as fh:
        txt = fh.read()
    parts = re.split(r"^t=([\d.]+)(?: phase=(\S+))?\n", txt, flags=re.M)
    rows = []
    for i in range(1, len(parts), 3):
        body = parts[i + 2]
        if "{" not in body:
            continue
        try:
            g = json.loads(body[body.index("{"):])["gpu_data"][0]
        except (ValueError, KeyError, IndexError):
            continue
        clk = [v["clk"]["value"] for k, v in g.get("clock", {}).items()
               if k.startswith("gfx_") and isinstance(v.get("clk", {}).get("value"), (int, float))]
        pw = g.get("power", {}).get("socket_power", {}).get("value")
        if clk and isinstance(pw, (int, float)):
            rows.append((float(parts[i]), parts[i + 1] or "-", float(pw), sum(clk) / len(clk)))
    lines = ["| phase | busy samples | socket power W (median / max) | mean shader clock MHz (median) |",
             "|---|---|---|---|"]
    phases = []
    for r in rows:
        if r[1] not in phases:
            phases.append(r[1])
    for ph in phases:
        sel = [r for r in rows if r[1] == ph and r[3] > busy_mhz]
        if sel:
            lines.append("| %s | %d | %.0f / %.0f | %.0f |" % (ph, len(sel), statistics.median(r[2] for r in sel),
                                                              max(r[2] for r in sel), statistics.median(r[3] for r in sel)))
    idle = [r for r in rows if r[3] <= busy_mhz]
    if idle:
        lines.append("")
        lines.append("%d samples with the GPU idle (clocks below %.0f MHz): socket power median %.0f W." % (
            len(idle), busy_mhz, statistics.median(r[2] for r in idle)))
    return "\n".join(lines), rows


# ---------------------------------------------------------------- timing helpers

def _upload(inp):
    import torch
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        if v.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        out[k] = t.cuda()
    return out


def _time_steps(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(steps):
        fn()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _step_stats(fn, steps):
    """Median / min / max of single-step times (events around each step on the current stream)."""
    import torch
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(st)
    for i in range(steps):
        fn()
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return {"median": round(float(np.median(t)), 4), "min": round(float(t.min()), 4), "max": round(float(t.max()), 4)}


def _copy_gbs(nbytes=1 << 30, reps=5):
    """Device-to-device copy bandwidth (read + write bytes per second): HBM context for decode."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _kernel_times(fn, steps):
    """Average duration per launch of each kernel class, from HIP events the library records
    on the launch stream around every kernel."""
    import torch
    import fine_grained_shared_amd as moe
    torch.cuda.synchronize()
    moe.moe_profile_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    moe.moe_profile_enable(False)
    res = {}
    for k, name in enumerate(moe.PROF_NAMES):
        n, ms = moe.moe_profile_query(k)
        if n:
            res[name] = {"launches_per_step": n / steps, "ms_per_step": ms / steps}
    return res


def _scrubbed_step_ms(fn, steps, scrub):
    """Average time of fn over `steps` calls, each after a write over `scrub` (a device buffer larger
    than the 256 MB last-level cache), with events around fn only: every call starts from cold caches."""
    import torch
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        scrub.fill_(i & 0xFF)
        ev[i][0].record(st)
        fn()
        ev[i][1].record(st)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def _layer_call(w, d, flags, T=None, bias="default"):
    """A closure running moe_layer_forward on the first T tokens of the uploaded inputs d."""
    import torch
    import fine_grained_shared_amd as moe
    T = w.T if T is None else T
    shape = moe.make_shape(T, w.H, w.N_r, w.K_r, w.Ks, w.I, w.gating, w.act, w.dtype)
    ws = moe.workspace(shape)
    u = d["u"] if T == w.T else d["u"][:T].contiguous()
    out = torch.empty((T, w.H), dtype=moe.torch_dtype(shape), device="cuda")
    idx = torch.empty((T, max(w.K_r, 1)), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, max(w.K_r, 1)), dtype=torch.float32, device="cuda")
    b = d["bias"] if bias == "default" else bias

    def fn():
        moe.moe_layer_forward(shape, u, d["centroids"], b, d["w1"], d["b1"], d["w2"], d["w1_sh"], d["b1_sh"],
                              d["w2_sh"], flags, out, idx, wts, ws)
    return fn, idx


def _pack_all(w, d):
    """Routed banks and the shared gate/up bank in fragment order (bf16 layers); returns the flags."""
    import fine_grained_shared_amd as moe
    if w.dtype != 1:
        return 0
    for k in ("w1", "w2") + (("w1_sh",) if w.Ks > 0 else ()):
        d[k] = moe.pack_weights(d[k])
    return moe.MOE_FLAG_PACKED_WEIGHTS | (moe.MOE_FLAG_PACKED_SHARED_UP if w.Ks > 0 else 0)


def other_workloads(steps, warmup, names=("c1a", "c1b", "c1b_iso", "c2", "c4p")):
    """The other prefill layers of the workload table, timed like the headline one, and the
    high-sparsity decode slice (the first 64 tokens of its prefill inputs) with the caches scrubbed
    before every step (its touched weights, about 0.26 GB, would otherwise stay in the 256 MB
    last-level cache from one step to the next)."""
    import torch
    import synth
    res = {}
    for name in names:
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w)
        d = _upload(inp)
        del inp
        flags = _pack_all(w, d)
        fn, idx = _layer_call(w, d, flags)
        ms = _time_steps(fn, steps, warmup)
        kt = _kernel_times(fn, max(2, min(steps, 10)))
        fl = layer_flops(w)
        counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.N_r)
        res[name] = {"workload": w.desc, "ms_per_step": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
                     "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                     "pct_bf16_peak": round(100 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in kt.items()},
                     "load_max_over_mean": round(float(counts.max() / counts.mean()), 2),
                     "empty_experts": int((counts == 0).sum())}
        print("[bench] %s prefill %.3f ms/step, %.1f %% of bf16 peak" % (name, ms, res[name]["pct_bf16_peak"]),
              file=sys.stderr, flush=True)
        if name == "c4p":
            Td = synth.WORKLOADS["c4d"].T
            wd = w.with_(T=Td)
            dfn, didx = _layer_call(w, d, flags, T=Td)
            for _ in range(warmup):
                dfn()
            scrub = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
            cold = _scrubbed_step_ms(dfn, max(steps, 10), scrub)
            warm = _time_steps(dfn, max(steps, 10), warmup)
            dkt = _kernel_times(dfn, 10)
            del scrub
            touched = int(np.unique(didx.cpu().numpy()).size)
            nb = decode_bytes(wd, touched)
            res["c4d"] = {"workload": synth.WORKLOADS["c4d"].desc, "ms_per_step": round(cold, 4),
                          "tokens_per_s": round(Td / (cold * 1e-3), 1), "touched_experts": touched,
                          "algorithmic_bytes": nb, "GB_per_s": round(nb / (cold * 1e-3) / 1e9, 1),
                          "pct_hbm_peak": round(100 * nb / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                          "cache": "1 GiB scrub written before every timed step (events around the step only)",
                          "warm_cache_ms_per_step": round(warm, 4),
                          "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in dkt.items()}}
            print("[bench] c4d decode %.4f ms/step (cold caches), %.4f warm" % (cold, warm), file=sys.stderr,
                  flush=True)
        d.clear()
        torch.cuda.empty_cache()
    return res


def cpu_baseline(w, inp, budget_s=20.0):
    """The fp64 oracle on the host cores, on a bounded sample of the workload's tokens."""
    import oracle
    s = oracle.shape_of(w)
    probe = np.arange(0, w.T, max(1, w.T // 8))[:8].astype(np.int64)
    t0 = time.time()
    oracle.layer(s, inp, tokens=probe)
    per_tok = max((time.time() - t0) / len(probe), 1e-6)
    n = int(min(max(budget_s / per_tok, 8), w.T))
    toks = np.linspace(0, w.T - 1, n).astype(np.int64)
    t0 = time.time()
    oracle.layer(s, inp, tokens=toks)
    dt = time.time() - t0
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "%d of %d tokens (evenly strided) of the same layer, full forward in fp64, %.1f s" % (
                n, w.T, dt),
            "cpu_model": _cpu_model(), "fp64_gflops": round(layer_flops(w) / w.T * n / dt / 1e9, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3p")
    ap.add_argument("--decode-tokens", type=int, default=128)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the other workloads of the table")
    ap.add_argument("--no-unpacked", action="store_true",
                    help="with packed weights, skip timing the same step on the [out, in] banks")
    ap.add_argument("--rocprof-summary", metavar="TRACE_DIR", help="summarise a rocprofv3 run and exit")
    ap.add_argument("--pmc-fetch", metavar="DIR")
    ap.add_argument("--pmc-write", metavar="DIR")
    ap.add_argument("--traffic-json", metavar="FILE")
    ap.add_argument("--counter-summary", metavar="PMC_DIR",
                    help="per-kernel MFMA busy %%, shader clock and HBM bytes of rocprofv3 --pmc runs, then exit")
    ap.add_argument("--pmc-rdreq", metavar="DIR", help="a TCC_EA0_RDREQ*_sum run for --counter-summary")
    ap.add_argument("--power-summary", metavar="LOG",
                    help="socket power and shader clocks from a log of amd-smi metric samples, then exit")
    ap.add_argument("--weights", choices=("packed", "unpacked"), default="packed",
                    help="routed expert banks in fragment order (moe_pack_weights, done once when the weights "
                         "are loaded, before timing; the layer's output is bit-identical) or in the [out, in] "
                         "layout")
    args = ap.parse_args()
    if args.counter_summary:
        text, _ = counter_summary(args.counter_summary, args.pmc_fetch, args.pmc_write, rdreq_dir=args.pmc_rdreq)
        print(text)
        return
    if args.power_summary:
        print(power_summary(args.power_summary)[0])
        return
    if args.rocprof_summary:
        text, _ = rocprof_summary(args.rocprof_summary, args.pmc_fetch, args.pmc_write, args.traffic_json,
                                  dominant_kernel(args.weights == "packed"))
        print(text)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer runs data-parallel over tokens with replicated "
              "weights, so no exchange is needed and N>1 is not measured here (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import fine_grained_shared_amd as moe
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.load()
    w = synth.WORKLOADS[args.workload]
    t0 = time.time()
    inp = synth.make_inputs(w)
    gen_s = time.time() - t0
    d = _upload(inp)
    flags = 0
    unpacked = None
    if args.weights == "packed":
        # a storage layout of the same weights, made once when they are loaded (not part of a step);
        # the [out, in] banks are kept to time the same step on them as well
        packed_keys = ("w1", "w2") + (("w1_sh",) if w.Ks > 0 else ())
        unpacked = None if args.no_unpacked else {k: d[k] for k in packed_keys}
        for k in packed_keys:
            d[k] = moe.pack_weights(d[k])
        flags = moe.MOE_FLAG_PACKED_WEIGHTS | (moe.MOE_FLAG_PACKED_SHARED_UP if w.Ks > 0 else 0)
    torch.cuda.synchronize()
    print("[bench] inputs generated in %.1f s and uploaded (%s routed banks)" % (gen_s, args.weights),
          file=sys.stderr, flush=True)

    # plain 1 GiB device copy: reference point for the HBM byte counters of a profiled run
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    del src, dst

    shape = moe.make_shape(w.T, w.H, w.N_r, w.K_r, w.Ks, w.I, w.gating, w.act, w.dtype)
    ws = moe.workspace(shape)
    out = torch.empty((w.T, w.H), dtype=moe.torch_dtype(shape), device="cuda")
    idx = torch.empty((w.T, w.K_r), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.K_r), dtype=torch.float32, device="cuda")

    def step():
        moe.moe_layer_forward(shape, d["u"], d["centroids"], d["bias"], d["w1"], d["b1"], d["w2"], d["w1_sh"],
                              d["b1_sh"], d["w2_sh"], flags, out, idx, wts, ws)

    ms = _time_steps(step, args.steps, args.warmup)
    print("[bench] prefill %.3f ms/step" % ms, file=sys.stderr, flush=True)
    stats = _step_stats(step, args.steps)
    kt = _kernel_times(step, max(2, min(args.steps, 10)))
    flops = layer_flops(w)
    up = kt.get("ffn_up", {"ms_per_step": float("nan"), "launches_per_step": 1})
    up_ms = up["ms_per_step"] / up["launches_per_step"]
    up_tflops = routed_up_flops(w) / (up_ms * 1e-3) / 1e12
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.N_r)

    result = {
        "metric": METRIC,
        "value": round(w.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights, N(0,1/H) centroids, bias N(0,0.01))",
        "config": {"workload": w.desc, "T": w.T, "H": w.H, "N_r": w.N_r, "K_r": w.K_r, "Ks": w.Ks, "I": w.I,
                   "gating": "sigmoid+selection bias, normalised over selected",
                   "act": "SwiGLU", "parallelism": "single GPU",
                   "routed_weights": "fragment order (packed once at load)" if flags else "[out, in]",
                   "shared_up_weights": ("fragment order (packed once at load)"
                                         if flags & moe.MOE_FLAG_PACKED_SHARED_UP else "[out, in]")},
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": {"kernel": "routed expert gate/up grouped GEMM + SwiGLU (%s)" % dominant_kernel(flags),
                     "bound": "mfma", "achieved": round(up_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(up_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dominant_kernel(flags)),
                     "avg_launch_ms": round(up_ms, 4),
                     "algorithmic_flops_per_launch": routed_up_flops(w)},
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in kt.items()},
        "load": {"touched": int((counts > 0).sum()), "empty": int((counts == 0).sum()),
                 "max_over_mean": round(float(counts.max() / counts.mean()), 2)},
    }

    if unpacked is not None:
        def ustep():
            moe.moe_layer_forward(shape, d["u"], d["centroids"], d["bias"], unpacked["w1"], d["b1"], unpacked["w2"],
                                  unpacked.get("w1_sh", d["w1_sh"]), d["b1_sh"], d["w2_sh"], 0, out, idx, wts, ws)

        ums = _time_steps(ustep, max(5, args.steps // 2), args.warmup)
        result["unpacked_weights"] = {"ms_per_step": round(ums, 4), "value": round(w.T / (ums * 1e-3), 1),
                                      "note": "the same step on the [out, in] banks (bit-identical output)"}
        print("[bench] prefill, [out, in] routed banks: %.3f ms/step" % ums, file=sys.stderr, flush=True)
        del unpacked
        torch.cuda.empty_cache()

    if not args.no_decode:
        Td = args.decode_tokens
        print("[bench] timing decode, T=%d" % Td, file=sys.stderr, flush=True)
        wd = w.with_(T=Td)
        sd = moe.make_shape(Td, w.H, w.N_r, w.K_r, w.Ks, w.I, w.gating, w.act, w.dtype)
        wsd = moe.workspace(sd)
        ud = d["u"][:Td].contiguous()
        outd = torch.empty((Td, w.H), dtype=moe.torch_dtype(sd), device="cuda")
        idxd = torch.empty((Td, w.K_r), dtype=torch.int32, device="cuda")
        wtd = torch.empty((Td, w.K_r), dtype=torch.float32, device="cuda")

        def dstep():
            moe.moe_layer_forward(sd, ud, d["centroids"], d["bias"], d["w1"], d["b1"], d["w2"], d["w1_sh"],
                                  d["b1_sh"], d["w2_sh"], flags, outd, idxd, wtd, wsd)

        dms = _time_steps(dstep, max(args.steps, 10), args.warmup)
        dstats = _step_stats(dstep, max(args.steps, 10))
        dkt = _kernel_times(dstep, 10)
        copy = _copy_gbs()
        touched = int(np.unique(idxd.cpu().numpy()).size)
        nbytes = decode_bytes(wd, touched)
        gbs = nbytes / (dms * 1e-3) / 1e9
        result["decode"] = {"T": Td, "ms_per_step": round(dms, 4), "tokens_per_s": round(Td / (dms * 1e-3), 1),
                            "touched_experts": touched, "algorithmic_bytes": nbytes, "GB_per_s": round(gbs, 1),
                            "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2), "step_ms": dstats,
                            "copy_GB_per_s": round(copy, 1),
                            "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in dkt.items()}}
        print("[bench] decode %.3f ms/step, %.0f GB/s" % (dms, gbs), file=sys.stderr, flush=True)
        if w.gating == 1:
            # sensitivity: the selection bias set to 0 (near-uniform routing touches almost every expert)
            print("[bench] timing decode with the selection bias set to 0", file=sys.stderr, flush=True)
            zfn, zidx = _layer_call(w, d, flags, T=Td, bias=None)
            zms = _time_steps(zfn, max(args.steps, 10), args.warmup)
            zt = int(np.unique(zidx.cpu().numpy()).size)
            zb = decode_bytes(wd, zt)
            result["decode_bias0"] = {"T": Td, "bias": "0 (sensitivity run)", "ms_per_step": round(zms, 4),
                                      "touched_experts": zt, "algorithmic_bytes": zb,
                                      "GB_per_s": round(zb / (zms * 1e-3) / 1e9, 1),
                                      "pct_hbm_peak": round(100 * zb / (zms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
            print("[bench] decode, bias 0: %.3f ms/step, %d experts" % (zms, zt), file=sys.stderr, flush=True)

    if not args.no_other and args.workload == "c3p":
        d.clear()
        torch.cuda.empty_cache()
        result["other_workloads"] = other_workloads(args.steps, args.warmup)

    if not args.no_cpu:
        print("[bench] timing the fp64 oracle on the host cores", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, inp)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
