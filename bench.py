"""Benchmark of the Beam-shaped NVFP4 / FP8 routed-expert MoE layer on one MI355X.

One step = the whole hot path on one batch with inputs resident in HBM:
group-limited sigmoid routing + activation quantization + expert MLP
(permutation, gate/up GEMM + SwiGLU, h re-quantization, down GEMM, combine).
Offline weight quantization happens once before timing.

The headline line (``value``) is the 64-token decode layer in NVFP4 (hidden
5120, 256 experts, 8 groups of 32, keep 4, top 8, intermediate 2560); the same
run also measures the 8192-token prefill layer (Zipf-skewed router) and reports
it under ``prefill_8192``.  Per-kernel times come from hipEvents recorded at
the library's stage boundaries on the launch stream.

The default run also reports the FP8 layers (decode and prefill), the
standalone 32768 x 5120 NVFP4 quantize, the 4-layer stack in both formats, the
measured HBM-read and FP16-MFMA ceilings of this GPU, and the CPU oracle on
bounded samples (all host threads and one thread).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--fmt nvfp4|fp8|w4a16]
                       [--workload decode|prefill|stack|dense-fp8] [--no-prefill] [--no-extras]
                       [--no-cpu-baseline] [--ceilings]
"""

import argparse
import dataclasses
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_scaled_fp4_sigmoid_amd as bsm  # noqa: E402
import workloads as W  # noqa: E402

METRIC = "MoE-layer tokens/s + TFLOP/s & HBM GB/s (% roofline), decode-64 & prefill-8192"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "f16": 2500.0}
NVFP4_BYTES_PER_WEIGHT = 0.5625  # 4-bit code + one 1-byte E4M3 scale per 16 values


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its launch stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h.value)

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return float(out.value)

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "moe_decode64_nvfp4_traffic.json")
GEMM_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_scaled_fp4_sigmoid_amd", "csrc", "bsm_moe.hip")
COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read and 1 GiB written


def _source_digest():
    """SHA-256 of the kernel source's code: comments and blank space are dropped, so editing only
    comments keeps the counter record valid (the source holds no string literal with //)."""
    import hashlib
    import re
    with open(GEMM_SOURCE) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(" ".join(line.split()) for line in src.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()


def copy_calibration(dev):
    """A plain elementwise copy of known size (1 GiB in, 1 GiB out) for scaling the HBM counters."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def _pmc_per_kernel(path):
    """{kernel name: [counter value per dispatch]} from a rocprofv3 counter-collection CSV."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _kernel_label(name):
    """Library kernel name with its template arguments, from a demangled or mangled name; None otherwise."""
    import re
    m = re.search(r'bsm::\(anonymous namespace\)::(k_[a-z0-9_]+)(<([^>]*)>)?', name)
    if m:
        args = m.group(3).replace(' ', '') if m.group(3) else ''
        return m.group(1) + (f"<{args}>" if args else "")
    m = re.search(r'\d+(k_[a-z0-9_]+)(I(.*?E)EE|E)', name)
    if not m or not name.startswith('_ZN3bsm'):
        return None
    args = []
    if m.group(3):
        for kind, val in re.findall(r'L([bi])(\d+)E', m.group(3)):
            args.append(('true' if val == '1' else 'false') if kind == 'b' else val)
    return m.group(1) + (f"<{','.join(args)}>" if args else "")


def summarize_trace(trace_csv, title, command, notes=()):
    """Print a rocprofv3 kernel_trace.csv as library kernels grouped by (name, template arguments, grid)."""
    import csv
    from collections import defaultdict
    groups = defaultdict(list)
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            k = _kernel_label(r['Kernel_Name'])
            if not k:
                continue
            grid = f"{int(r['Grid_Size_X']) // int(r['Workgroup_Size_X'])}x{r['Grid_Size_Y']}x{r['Grid_Size_Z']}"
            groups[(k, grid)].append((int(r['End_Timestamp']) - int(r['Start_Timestamp'])) / 1e3)
    print(f"# {title}")
    print(f"# command: {command}")
    print(f"# summary: python3 bench.py --summarize-trace <kernel_trace.csv> '<title>' '<command>'")
    print("# rocprofv3 kernel trace, library kernels grouped by kernel, template arguments and grid (workgroups);")
    print("# torch kernels of input generation omitted.  Durations in microseconds.")
    for n in notes:
        print(f"# {n}")
    print(f"{'kernel':40s} {'grid':>14s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
    for (k, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"{k:40s} {grid:>14s} {len(v):6d} {sum(v) / len(v):10.2f} {min(v):10.2f} {max(v):10.2f}")


def summarize_pmc(fetch_csv, write_csv, command, bench_json=None):
    """Turn the FETCH_SIZE and WRITE_SIZE runs into HBM bytes per gate/up GEMM launch.

    Writes the JSON record that bench.py reads back and a text summary beside it;
    ``bench_json`` (a default bench run's output line) supplies the algorithmic bytes.
    """
    fetch, write = _pmc_per_kernel(fetch_csv), _pmc_per_kernel(write_csv)

    def pick(d, pred):
        keys = [k for k in d if pred(k)]
        assert keys, "kernel not found in the counter CSV"
        return max(keys, key=lambda k: len(d[k]))

    # the decode gate/up kernel: the chunk-staged NVFP4 one, else the per-super-step one
    rows = [k for k in fetch if "k_skinny_rowsILb1ELb1ELi2ELb0E" in k]  # <NVFP4, gate/up, NT 2, not W4A16>
    gemm = pick(fetch, (lambda k: k in rows) if rows else (lambda k: "k_skinny" in k and "ILb1ELb1ELi128" in k))
    label = _kernel_label(gemm) or gemm[:60]
    copyk = max((k for k in fetch if "elementwise" in k or "vectorized" in k), key=lambda k: max(fetch[k]))
    f_copy, w_copy = max(fetch[copyk]), max(write[copyk])
    sf, sw = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    fb = float(np.mean(fetch[gemm])) * sf
    wb = float(np.mean(write[gemm])) * sw
    res = {"kernel": label + " gate/up (decode-64 NVFP4)", "dispatches": len(fetch[gemm]),
           "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb, "traffic_bytes_per_launch": fb + wb,
           "copy_kernel": copyk[:80], "copy_counter_fetch": f_copy, "copy_counter_write": w_copy,
           "scale_fetch": sf, "scale_write": sw, "gemm_source_sha256": _source_digest(), "command": command}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(res, f, indent=1)
    alg = None
    if bench_json and os.path.exists(bench_json):
        with open(bench_json) as f:
            alg = json.loads(f.readline())["roofline"]["algorithmic_bytes_per_launch"]
    write_traffic_text(res, alg)
    print(json.dumps(res, indent=1))


def write_traffic_text(res, alg=None):
    """The text summary beside the traffic record (``alg``: the algorithmic bytes per launch, if known)."""
    command, label = res["command"], res["kernel"].split(" ")[0]
    f_copy, w_copy, fb, wb = res["copy_counter_fetch"], res["copy_counter_write"], res["fetch_bytes_per_launch"], \
        res["write_bytes_per_launch"]
    lines = [
        f"# HBM traffic of the gate/up GEMM ({label}) at decode-64 NVFP4, MI355X",
        "# command (two runs, one counter each):",
        "#   " + command.replace(" (then WRITE_SIZE)", "").replace("fetch|write", "fetch"),
        "#   " + command.replace("FETCH_SIZE (then WRITE_SIZE)", "WRITE_SIZE").replace("fetch|write", "write"),
        "#   python3 bench.py --summarize-pmc <fetch counter_collection.csv> <write counter_collection.csv> "
        "'<command>' <bench.py output line>",
        "# scaling: the same counters on a 1 GiB elementwise copy (torch.add(src, 0, out=dst), 1 GiB read + 1 GiB "
        "written)",
        f"copy kernel FETCH_SIZE counter      {f_copy:.1f}  -> {res['scale_fetch']:.2f} bytes per unit",
        f"copy kernel WRITE_SIZE counter      {w_copy:.1f}  -> {res['scale_write']:.2f} bytes per unit",
        f"gate/up dispatches measured          {res['dispatches']}",
        f"fetched bytes per launch             {fb:.4g}",
        f"written bytes per launch             {wb:.4g}",
        f"HBM traffic per launch               {fb + wb:.4g}",
    ]
    if alg:
        lines += [f"algorithmic bytes per launch         {alg:.4g}  (active experts x 14,745,600 B of gate/up "
                  "weights + x codes/scales + h written)",
                  f"traffic / algorithmic                {(fb + wb) / alg:.3f}"]
    lines.append("# FETCH_SIZE counts what L2 requests from the memory fabric, so Infinity Cache hits are included "
                 "in it.")
    with open(TRAFFIC_FILE[:-len(".json")] + ".txt", "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_counters(title, command, kernel_filter, csvs):
    """Per-kernel averages of rocprofv3 --pmc runs (several counters per run), for the library kernels
    whose label contains ``kernel_filter``, with the derived ratios used in the design notes."""
    import csv
    from collections import defaultdict
    vals = defaultdict(list)
    for path in csvs:
        with open(path) as f:
            for r in csv.DictReader(f):
                k = _kernel_label(r["Kernel_Name"])
                if not k or kernel_filter not in k:
                    continue
                vals[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
    kernels = sorted({k for k, _ in vals})
    print(f"# {title}")
    print(f"# command (one run per counter set): {command}")
    print("# rocprofv3 --pmc counter collection, averages per dispatch (counters summed over the chip)")
    for k in kernels:
        c = {n: float(np.mean(v)) for (kk, n), v in vals.items() if kk == k}
        n_disp = max(len(v) for (kk, _), v in vals.items() if kk == k)
        print(f"\n## {k}  ({n_disp} dispatches)")
        for n in sorted(c):
            print(f"{n:32s} {c[n]:20.6g}")
        d = {}
        if "SQ_INSTS_VALU" in c and "SQ_INSTS_MFMA" in c and c["SQ_INSTS_MFMA"]:
            d["VALU instructions per MFMA"] = c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"]
        if "SQ_INSTS_LDS" in c and "SQ_INSTS_MFMA" in c and c["SQ_INSTS_MFMA"]:
            d["LDS instructions per MFMA"] = c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"]
        if "SQ_WAVE_CYCLES" in c and c["SQ_WAVE_CYCLES"]:
            for n in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VALU",
                      "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_ANY"):
                if n in c:
                    d[f"{n} / SQ_WAVE_CYCLES"] = c[n] / c["SQ_WAVE_CYCLES"]
        if "SQ_LDS_BANK_CONFLICT" in c and "SQ_ACTIVE_INST_LDS" in c and c["SQ_ACTIVE_INST_LDS"]:
            d["LDS bank-conflict cycles / LDS active cycles"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"]
        if d:
            print("# derived")
            for n, v in d.items():
                print(f"{n:48s} {v:10.4f}")


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter runs, if they match this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t["traffic_bytes_per_launch"] if t.get("gemm_source_sha256") == _source_digest() else None


def build_layer(cfg, fmt, dev):
    x = torch.from_numpy(W.activations(cfg)).to(dev, torch.bfloat16)
    wr = torch.from_numpy(W.router_weights(cfg)).to(dev, torch.bfloat16)
    w13, w2 = W.expert_weights_device(cfg, device=dev)
    # quantized offline, then the codes put in the pair layout the expert GEMMs read directly (same codes)
    weights = bsm.to_pair_layout(bsm.quantize_expert_weights(w13, w2, "fp8" if fmt == "fp8" else "nvfp4"))
    torch.cuda.synchronize()
    return x, wr, w13, w2, weights


def second_copy(x, wr, weights):
    """A second, separately allocated copy of a layer's inputs and weights.

    Steps alternate between the two copies, so a step never finds its inputs in
    the 256 MB Infinity Cache from the step before (the layer reads several GB).
    """
    w2 = dataclasses.replace(weights, **{f.name: getattr(weights, f.name).clone() for f in dataclasses.fields(weights)
                                         if isinstance(getattr(weights, f.name), torch.Tensor)})
    return x.clone(), wr.clone(), w2


def run_steps(cfg, fmt, x, wr, weights, steps, warmup, copies=None):
    """Time ``steps`` whole-path steps.

    ``copies``: optional further (x, wr, weights) copies; step i uses copy i mod n.
    Timed pass: the library records only the two stage events around the gate/up
    GEMM (its per-launch duration, for the roofline) on its launch stream.  A
    second, untimed pass records every stage boundary for the per-stage
    breakdown (each recorded event costs a few microseconds of GPU time).
    Returns (ms per step, per-stage ms, gate/up GEMM ms in the timed pass, counts); the per-stage
    dict also carries ``host_submit``, the host time per timed step spent submitting the work (a step
    whose GPU time is close to it is bound by the host).
    """
    T = x.shape[0]
    out = torch.empty((T, cfg.H), dtype=torch.float32, device=x.device)
    ws = None
    sets = [(x, wr, weights)] + list(copies or [])
    it = [0]

    def step():
        nonlocal ws
        x, wr, weights = sets[it[0] % len(sets)]
        it[0] += 1
        if fmt == "nvfp4":  # routing and the quantization of x in one call (one pass of max|x| fewer)
            ids, wts, xq = bsm.route_nvfp4_quantize(x, wr, cfg.n_group, cfg.topk_group, cfg.topk)
        else:
            ids, wts = bsm.route(x, wr, cfg.n_group, cfg.topk_group, cfg.topk)
        if fmt == "w4a16":  # weight-only: the BF16 activations go in as they are
            o, ws = bsm.moe_expert_mlp_w4a16(weights, x, ids, wts, cfg.combine_scale, out=out, ws=ws,
                                             return_workspace=True)
            return ids
        if fmt != "nvfp4":
            xq = bsm.quantize_activations(x, fmt)
        o, ws = bsm.moe_expert_mlp(weights, xq, ids, wts, cfg.combine_scale, out=out, ws=ws, return_workspace=True)
        return ids

    for _ in range(warmup):
        ids = step()
    torch.cuda.synchronize()
    ev = HipEvents(2 * steps)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    h0 = time.perf_counter()
    for i in range(steps):
        bsm.set_stage_events(0, [None, ev.ev[2 * i], ev.ev[2 * i + 1], None, None, None])
        ids = step()
    host_ms = (time.perf_counter() - h0) * 1e3 / steps
    stop.record()
    torch.cuda.synchronize()
    bsm.set_stage_events(0, [])
    total_ms = start.elapsed_time(stop)
    g1_ms = float(np.mean([ev.ms(2 * i, 2 * i + 1) for i in range(steps)]))
    ev.close()

    ev = HipEvents(steps * 6 + steps * 3)
    for i in range(steps):
        bsm.set_stage_events(1, ev.ev[steps * 6 + 3 * i: steps * 6 + 3 * i + 3])
        bsm.set_stage_events(0, ev.ev[6 * i: 6 * i + 6])
        step()
    torch.cuda.synchronize()
    bsm.set_stage_events(0, [])
    bsm.set_stage_events(1, [])
    stages = {k: [] for k in ("route", "route_select", "permute", "gemm1", "hquant", "gemm2", "combine")}
    for i in range(steps):
        b = 6 * i
        r = steps * 6 + 3 * i
        stages["route"].append(ev.ms(r, r + 2))
        stages["route_select"].append(ev.ms(r + 1, r + 2))
        stages["permute"].append(ev.ms(b, b + 1))
        stages["gemm1"].append(ev.ms(b + 1, b + 2))
        stages["hquant"].append(ev.ms(b + 2, b + 3))
        stages["gemm2"].append(ev.ms(b + 3, b + 4))
        stages["combine"].append(ev.ms(b + 4, b + 5))
    ev.close()
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=cfg.E)
    stage_ms = {k: float(np.mean(v)) for k, v in stages.items()}
    stage_ms["host_submit"] = host_ms  # host time to submit one timed step (not a GPU stage)
    return total_ms / steps, stage_ms, g1_ms, counts


def layer_numbers(cfg, fmt, T, ms, stage_ms, g1_ms, counts):
    P = T * cfg.topk
    n_act = int((counts > 0).sum())
    flop = 2.0 * P * 3 * cfg.H * cfg.I + 2.0 * T * cfg.E * cfg.H
    nv = fmt != "fp8"  # NVFP4 weights (W4A4 and weight-only W4A16)
    wbytes_per_expert = 3 * cfg.H * cfg.I * (NVFP4_BYTES_PER_WEIGHT if nv else 1.0) + \
        (0 if nv else 4 * (2 * cfg.I + cfg.H))
    layer_bytes = n_act * wbytes_per_expert + T * cfg.H * 2 + cfg.E * cfg.H * 2 + T * cfg.H * 4
    # dominant kernel: gate/up GEMM.  Algorithmic bytes per launch: the gate+up weights of
    # every active expert, the quantized activations it reads, the FP32 h it writes.
    g1_w = 2 * cfg.I * cfg.H * (NVFP4_BYTES_PER_WEIGHT if nv else 1.0) + (0 if nv else 4 * 2 * cfg.I)
    x_b = {"nvfp4": NVFP4_BYTES_PER_WEIGHT, "fp8": 1.0, "w4a16": 2.0}[fmt]
    g1_bytes = n_act * g1_w + T * cfg.H * x_b + P * cfg.I * 4
    g1_flop = 2.0 * P * 2 * cfg.I * cfg.H
    return {
        "tokens_per_s": T / (ms * 1e-3),
        "ms_per_step": ms,
        "tflops": flop / (ms * 1e-3) / 1e12,
        "gbps": layer_bytes / (ms * 1e-3) / 1e9,
        "hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "active_experts": n_act,
        "max_expert_rows": int(counts.max()),
        "layer_flop": flop,
        "layer_bytes": layer_bytes,
        "stage_ms": stage_ms,
        "gemm1": {"ms": g1_ms, "bytes": g1_bytes, "flop": g1_flop,
                  "gbps": g1_bytes / (g1_ms * 1e-3) / 1e9, "tflops": g1_flop / (g1_ms * 1e-3) / 1e12},
    }


def _blas_info():
    """BLAS library, version and thread count numpy uses, and the numpy version."""
    try:
        import threadpoolctl
        info = [d for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
        blas = {k: info[0].get(k) for k in ("internal_api", "version", "num_threads")} if info else None
    except ImportError:
        blas = None
    return {"numpy": np.__version__, "blas": blas}


def _thread_limit(n):
    import contextlib
    try:
        import threadpoolctl
        return threadpoolctl.threadpool_limits(n)
    except ImportError:
        return contextlib.nullcontext()


def _oracle_decode_time(cfg, fmt, x_np, wr_np, ids, wts, experts, sample):
    """Seconds the oracle takes for the whole decode layer: routing and activation quantization of every
    token are timed whole; the expert MLP is timed on ``sample`` pairs (one token's first slots, one expert
    each) and scaled by the layer's active experts, since the oracle's per-expert work (decoding the
    expert's weights exactly, its GEMMs) dominates and does not depend on the rows at decode."""
    from oracle import moe as OM
    from oracle import route as OR

    t0 = time.perf_counter()
    OR.route(x_np, wr_np, cfg.n_group, cfg.topk_group, cfg.topk)
    t_route = time.perf_counter() - t0
    t0 = time.perf_counter()
    OM.quantize_activations(x_np, fmt)
    t_xq = time.perf_counter() - t0
    _, xh = OM.quantize_activations(x_np[:1], fmt)
    t0 = time.perf_counter()
    OM.moe_expert_mlp(xh, ids[:1, :sample], wts[:1, :sample], experts, fmt, cfg.combine_scale)
    t_mlp = time.perf_counter() - t0
    n_act = len(np.unique(ids))
    return t_route + t_xq + t_mlp / sample * n_act, (t_route, t_xq, t_mlp, n_act)


def cpu_baseline(dev):
    """The CPU oracle (NumPy, float64 GEMMs on exactly decoded operands) on the host cores of this machine, on
    bounded samples, with all host threads and with one thread:

    * decode-64 NVFP4 (the headline workload): routing and activation quantization of all 64 tokens
      timed whole, the expert MLP timed on 4 experts and scaled per active expert (222);
    * the tiny layer (64 tokens, hidden 256, 16 experts): the whole layer;
    * the standalone 32768 x 5120 quantize: 512 rows, scaled by 64.

    Weight quantization is offline (untimed), as on the GPU."""
    from oracle import moe as OM
    from oracle import quant as Q
    from oracle import quant_c as QC
    from oracle import route as OR

    cfg = W.DECODE
    x_np, wr_np = W.activations(cfg), W.router_weights(cfg)
    ids, wts, _, _ = OR.route(x_np, wr_np, cfg.n_group, cfg.topk_group, cfg.topk)
    sample = 4
    es = [int(e) for e in ids[0, :sample]]
    w13, w2 = W.expert_weights_device(cfg, device=dev, experts=es)
    experts = {}
    for i, e in enumerate(es):
        bits = [t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                for t in (w13[i, :cfg.I], w13[i, cfg.I:], w2[i])]
        ex = OM.NVFP4Expert(*bits, q=QC)  # offline quantization (untimed) by the oracle's C loops ...
        ex.q = Q  # ... and the timed decoding by its NumPy definition
        experts[e] = ex
    del w13, w2
    tcfg = W.TINY
    tx, twr = W.activations(tcfg), W.router_weights(tcfg)
    texperts = {e: OM.NVFP4Expert(*W.expert_weights_host(tcfg, e), q=QC) for e in range(tcfg.E)}
    for ex in texperts.values():
        ex.q = Q
    qx = W.quant_tensor_host((512, 5120), seed=2)

    def measure():
        t_dec, parts = _oracle_decode_time(cfg, "nvfp4", x_np, wr_np, ids, wts, experts, sample)
        t0 = time.perf_counter()
        OM.moe_layer(tx, twr, texperts, "nvfp4", tcfg.n_group, tcfg.topk_group, tcfg.topk, tcfg.combine_scale)
        t_tiny = time.perf_counter() - t0
        t0 = time.perf_counter()
        Q.nvfp4_quantize(qx)
        t_q = (time.perf_counter() - t0) * (W.QUANT_SHAPE[0] / qx.shape[0])
        return {"decode_tokens_per_s": cfg.T / t_dec, "decode_s": t_dec,
                "decode_parts_s": {"route": parts[0], "x_quant": parts[1], f"mlp_{sample}_experts": parts[2],
                                   "active_experts": parts[3]},
                "tiny_tokens_per_s": tcfg.T / t_tiny, "tiny_s": t_tiny,
                "quantize_32768x5120_s": t_q, "quantize_gbps": 429.9e6 / t_q / 1e9}

    threads = len(os.sched_getaffinity(0))
    full = measure()
    with _thread_limit(1):
        one = measure()
    def rnd(d):
        return {k: (round(v, 4) if isinstance(v, float) else rnd(v) if isinstance(v, dict) else v)
                for k, v in d.items()}

    return {"value": round(full["decode_tokens_per_s"], 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"decode-64 NVFP4 layer: routing + activation quantization of all 64 tokens timed whole, "
                       f"expert MLP of {sample} experts ({full['decode_parts_s'][f'mlp_{sample}_experts']:.2f} s) "
                       f"scaled to the {full['decode_parts_s']['active_experts']} active experts; NumPy float64 "
                       f"on {threads} host threads"),
            "all_threads": rnd(full), "one_thread": rnd(one), **_blas_info()}


def stack_numbers(dev, steps, warmup):
    """Four Beam-shaped MoE layers on a 4096-token FP32 stream (RMSNorm -> MoE -> depth-scaled residual),
    NVFP4 and FP8 side by side; one step = the whole 4-layer stack."""
    cfg = W.STACK
    x1 = torch.from_numpy(W.activations(cfg)).to(dev)
    res = {}
    for fmt in ("nvfp4", "fp8"):
        layers = []
        for li in range(cfg.layers):
            w13, w2 = W.expert_weights_device(cfg, layer=li, device=dev)
            wr = torch.from_numpy(W.router_weights(cfg, layer=li)).to(dev, torch.bfloat16)
            layers.append((wr, bsm.to_pair_layout(bsm.quantize_expert_weights(w13, w2, fmt))))
            del w13, w2
            torch.cuda.empty_cache()
        for _ in range(warmup):
            bsm.moe_stack(x1, layers, cfg.n_group, cfg.topk_group, cfg.topk)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            bsm.moe_stack(x1, layers, cfg.n_group, cfg.topk_group, cfg.topk)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / steps
        flop = cfg.layers * (2.0 * cfg.T * cfg.topk * 3 * cfg.H * cfg.I + 2.0 * cfg.T * cfg.E * cfg.H)
        wbytes = sum(sum(t.numel() * t.element_size() for t in (w.w13_codes, w.w13_scales, w.w2_codes, w.w2_scales))
                     for _, w in layers)
        res[fmt] = {"tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
                    "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                    "frac_f16_mfma_peak": round(flop / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["f16"], 4),
                    "weight_gbps": round(wbytes / (ms * 1e-3) / 1e9, 1)}
        print(f"[bench] stack {fmt}: {ms:.3f} ms per 4-layer step", file=sys.stderr, flush=True)
        del layers
        torch.cuda.empty_cache()
    return res


def run_stack(args, dev):
    """--workload stack: the 4-layer stack as the line's workload."""
    cfg = W.STACK
    res = stack_numbers(dev, args.steps, args.warmup)
    line = {
        "metric": METRIC, "value": res["nvfp4"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["nvfp4"]["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4-e2m1 (exact f16 mfma, f32 acc); fp8 alongside",
        "data": "synthetic (seeded Beam-shaped activations, router and expert weights)",
        "config": {"workload": "beam-stack-4x4096: 4 MoE layers, FP32 RMSNorm + depth-scaled residual",
                   "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "layers": cfg.layers, "topk": cfg.topk},
        "stack": res,
    }
    print(json.dumps(line))


def quantize_numbers(dev, steps, warmup):
    """The standalone NVFP4 quantize of a 32768 x 5120 bf16 tensor (Student-t with outlier rows): global
    amax, per-16 E4M3 scales and E2M1 codes; algorithmic bytes 2 B read + 0.5625 B written per value."""
    xs = [W.quant_tensor_device(device=dev), None]
    xs[1] = xs[0].clone()
    R, C = W.QUANT_SHAPE
    codes = torch.empty((R, C // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((R, C // 16), dtype=torch.uint8, device=dev)
    gs = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = None
    for i in range(warmup):
        ws = bsm.nvfp4_quantize_into(xs[i % 2], codes, scales, gs, ws)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        ws = bsm.nvfp4_quantize_into(xs[i % 2], codes, scales, gs, ws)
    stop.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) / steps * 1e3
    alg = R * C * 2 + R * C // 2 + R * C // 16
    return {"us": round(us, 2), "algorithmic_bytes": alg, "gbps": round(alg / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "floor_us": round(alg / (HBM_PEAK_GBS * 1e9) * 1e6, 2)}


def ceilings(dev, reps=10):
    """Measured ceilings of this GPU: streaming HBM read (best over workgroup counts) and the FP16 MFMA
    rate from registers (32x32x16 and 16x16x32, FP32 accumulation)."""
    nbytes = 4 << 30
    bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(2)]
    best = 0.0
    for wgs in (512, 768, 1024, 2048, 4096, 8192):
        sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
        bsm.ceiling_hbm_read(bufs[0], wgs, sink)
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for r in range(reps):
            bsm.ceiling_hbm_read(bufs[r % 2], wgs, sink)
        stop.record()
        torch.cuda.synchronize()
        best = max(best, nbytes * reps / (start.elapsed_time(stop) * 1e-3) / 1e9)
    del bufs
    torch.cuda.empty_cache()
    out = {"hbm_read_gbps": round(best, 1)}
    wgs, iters = 2048, 4000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    for shape, name, fl in ((0, "mfma_f16_32x32x16_tflops", 32768), (1, "mfma_f16_16x16x32_tflops", 16384)):
        bsm.ceiling_mfma_f16(shape, iters, wgs, sink)
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            bsm.ceiling_mfma_f16(shape, iters, wgs, sink)
        stop.record()
        torch.cuda.synchronize()
        flop = wgs * 4 * iters * 8 * fl * reps
        out[name] = round(flop / (start.elapsed_time(stop) * 1e-3) / 1e12, 1)
    return out


def run_dense_fp8(args, dev):
    """Dense FP8_DYNAMIC block at decode (64 tokens): attention q/k/v/gate/o projections and the dense
    SwiGLU MLP (hidden 5120, intermediate 20480), all W8A8 with per-channel / per-token scales."""
    T, H, I, NQ, NKV = 64, 5120, 20480, 6144, 1024
    gen = torch.Generator(device=dev)
    gen.manual_seed(5120)

    def w(n, k):
        return bsm.fp8_quantize((torch.randn((n, k), generator=gen, device=dev) * 0.02).to(torch.bfloat16))

    proj = {"q": w(NQ, H), "k": w(NKV, H), "v": w(NKV, H), "gate": w(NQ, H), "o": w(H, NQ)}
    w13 = (torch.randn((1, 2 * I, H), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((1, H, I), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    mlp = bsm.quantize_expert_weights(w13, w2, "fp8")
    del w13, w2
    x = torch.from_numpy(W.activations(W.DECODE)).to(dev, torch.bfloat16)
    outs = {k: torch.empty((T, v[0].shape[0]), dtype=torch.float32, device=dev) for k, v in proj.items()}
    mlp_out = torch.empty((T, H), dtype=torch.float32, device=dev)

    def step():
        xq = bsm.fp8_quantize(x)
        for k in ("q", "k", "v", "gate"):
            bsm.fp8_linear(xq, proj[k], out=outs[k])
        bsm.fp8_linear(bsm.fp8_quantize(outs["q"]), proj["o"], out=outs["o"])
        bsm.fp8_dense_mlp(mlp, x, out=mlp_out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    wbytes = sum(v[0].numel() + 4 * v[1].numel() for v in proj.values()) + \
        mlp.w13_codes.numel() + mlp.w2_codes.numel() + 4 * (mlp.w13_scales.numel() + mlp.w2_scales.numel())
    gbps = wbytes / (ms * 1e-3) / 1e9
    print(f"[bench] dense fp8 block: {ms:.3f} ms/step, {gbps:.0f} GB/s of weights", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "dense FP8_DYNAMIC block tokens/s (attention projections + dense MLP), decode-64",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8-e4m3 (exact f16 mfma, f32 acc)", "data": "synthetic",
        "config": {"workload": "beam dense fp8 block: q/k/v/gate/o projections + dense SwiGLU MLP, 64 tokens",
                   "T": T, "H": H, "I_dense": I, "q_heads": 48, "kv_heads": 8, "head_dim": 128},
        "gbps_weights": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBS, 4), "weight_bytes": int(wbytes)}))


def prefill_object(fmt, pn, pms, pst, psteps):
    mm = {"nvfp4": "fp4", "fp8": "fp8", "w4a16": "f16"}[fmt]
    return {
        "tokens_per_s": round(pn["tokens_per_s"], 1), "ms_per_step": round(pms, 4),
        "tflops": round(pn["tflops"], 2), "frac_fp4_or_fp8_peak": round(pn["tflops"] / PEAK_TFLOPS[mm], 4),
        "frac_f16_mfma_peak": round(pn["tflops"] / PEAK_TFLOPS["f16"], 4), "gbps": round(pn["gbps"], 1),
        "active_experts": pn["active_experts"], "max_expert_rows": pn["max_expert_rows"],
        "stage_ms": {k: round(v, 4) for k, v in pst.items()},
        "gemm1": {k: round(v, 3) for k, v in pn["gemm1"].items()},
        "steps": psteps,
    }


def measure_layer(cfg, fmt, dev, steps, warmup):
    x, wr, w13, w2, weights = build_layer(cfg, fmt, dev)
    del w13, w2
    torch.cuda.empty_cache()
    ms, stage_ms, g1_ms, counts = run_steps(cfg, fmt, x, wr, weights, steps, warmup,
                                            copies=[second_copy(x, wr, weights)])
    del x, wr, weights
    torch.cuda.empty_cache()
    print(f"[bench] {cfg.name} {fmt}: {ms:.3f} ms/step, stages {stage_ms}", file=sys.stderr, flush=True)
    return ms, stage_ms, g1_ms, layer_numbers(cfg, fmt, cfg.T, ms, stage_ms, g1_ms, counts)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--fmt", default="nvfp4", choices=["nvfp4", "fp8", "w4a16"])
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "prefill-uniform", "stack",
                                                               "dense-fp8"])
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the FP8 layers, the standalone quantize, the stack and the ceilings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ceilings", action="store_true", help="only measure the HBM read and FP16 MFMA ceilings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB elementwise copy (reference for the HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG",
                    help="FETCH_CSV WRITE_CSV COMMAND [BENCH_JSON]: write the gate/up GEMM HBM traffic from two "
                         "rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="TITLE COMMAND KERNEL_FILTER CSV [CSV ...]: print per-kernel averages of rocprofv3 --pmc "
                         "counter CSVs and exit")
    ap.add_argument("--summarize-trace", nargs="+", metavar="ARG",
                    help="KERNEL_TRACE_CSV TITLE COMMAND [NOTE ...]: print the kernel summary of a rocprofv3 "
                         "--kernel-trace run and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (3, 4):
            ap.error("--summarize-pmc needs FETCH_CSV WRITE_CSV COMMAND [BENCH_JSON]")
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_counters:
        if len(args.summarize_counters) < 4:
            ap.error("--summarize-counters needs TITLE COMMAND KERNEL_FILTER CSV [CSV ...]")
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.summarize_counters[2],
                           args.summarize_counters[3:])
        return
    if args.summarize_trace:
        if len(args.summarize_trace) < 3:
            ap.error("--summarize-trace needs KERNEL_TRACE_CSV TITLE COMMAND")
        summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.summarize_trace[2],
                        args.summarize_trace[3:])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs the MI355X"
    dev = torch.device("cuda:0")
    bsm.load()

    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(dev)}))
        return
    if args.workload == "stack":
        run_stack(args, dev)
        return
    if args.workload == "dense-fp8":
        run_dense_fp8(args, dev)
        return
    main_cfg = {"decode": W.DECODE, "prefill": W.PREFILL, "prefill-uniform": W.PREFILL_UNIFORM}[args.workload]
    ms, stage_ms, g1_ms, main_nums = measure_layer(main_cfg, args.fmt, dev, args.steps, args.warmup)

    g1 = main_nums["gemm1"]
    traffic = measured_traffic() if (args.workload == "decode" and args.fmt == "nvfp4") else None
    roofline = {"bound": "hbm", "achieved": round(g1["gbps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(g1["gbps"] / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else int(traffic), "traffic_unit": "bytes per launch",
                "kernel": "gate/up GEMM + SwiGLU",
                "algorithmic_bytes_per_launch": int(g1["bytes"]), "avg_launch_ms": round(g1["ms"], 4)}
    if args.copy_calibration:
        copy_calibration(dev)

    extras = args.workload == "decode" and not args.no_extras
    psteps = max(3, args.steps // 4)
    prefill = None
    if args.workload == "decode" and not args.no_prefill:
        pms, pst, _, pn = measure_layer(W.PREFILL, args.fmt, dev, psteps, 2)
        prefill = prefill_object(args.fmt, pn, pms, pst, psteps)

    fp8_decode = fp8_prefill = quant = stack = ceil = uniform = None
    if extras and not args.no_prefill:
        ums, ust, _, un = measure_layer(W.PREFILL_UNIFORM, args.fmt, dev, psteps, 2)
        uniform = prefill_object(args.fmt, un, ums, ust, psteps)
    if extras and args.fmt == "nvfp4":
        fms, fst, _, fn = measure_layer(W.DECODE, "fp8", dev, args.steps, args.warmup)
        fg1 = fn["gemm1"]
        fp8_decode = {"tokens_per_s": round(fn["tokens_per_s"], 1), "ms_per_step": round(fms, 4),
                      "gbps": round(fn["gbps"], 1), "hbm_frac": round(fn["hbm_frac"], 4),
                      "active_experts": fn["active_experts"], "stage_ms": {k: round(v, 4) for k, v in fst.items()},
                      "roofline_gate_up": {"bound": "hbm", "achieved": round(fg1["gbps"], 1), "peak": HBM_PEAK_GBS,
                                           "frac": round(fg1["gbps"] / HBM_PEAK_GBS, 4),
                                           "algorithmic_bytes_per_launch": int(fg1["bytes"]),
                                           "avg_launch_ms": round(fg1["ms"], 4)}}
        if not args.no_prefill:
            qms, qst, _, qn = measure_layer(W.PREFILL, "fp8", dev, psteps, 2)
            fp8_prefill = prefill_object("fp8", qn, qms, qst, psteps)
    if extras:
        quant = quantize_numbers(dev, args.steps, args.warmup)
        print(f"[bench] quantize 32768x5120: {quant}", file=sys.stderr, flush=True)
        stack = stack_numbers(dev, max(3, args.steps // 4), 2)
        ceil = ceilings(dev)
        print(f"[bench] ceilings: {ceil}", file=sys.stderr, flush=True)
        roofline["frac_of_measured_read_ceiling"] = round(g1["gbps"] / ceil["hbm_read_gbps"], 4)
        if prefill:
            prefill["frac_of_measured_f16_mfma_ceiling"] = round(
                prefill["tflops"] / ceil["mfma_f16_32x32x16_tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline and args.workload == "decode" and args.fmt == "nvfp4":
        cpu = cpu_baseline(dev)

    line = {
        "metric": METRIC,
        "value": round(main_nums["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"nvfp4": "nvfp4-e2m1 (exact f16 mfma, f32 acc)", "fp8": "fp8-e4m3 (exact f16 mfma, f32 acc)",
                  "w4a16": "nvfp4 weights, bf16 activations (exact bf16 mfma, f32 acc)"}[args.fmt],
        "data": "synthetic (seeded Beam-shaped activations, router and expert weights)",
        "config": {"workload": f"beam-{main_cfg.name}-{main_cfg.T} {args.fmt} MoE layer", "T": main_cfg.T,
                   "H": main_cfg.H, "I": main_cfg.I, "E": main_cfg.E, "n_group": main_cfg.n_group,
                   "topk_group": main_cfg.topk_group, "topk": main_cfg.topk, "combine_scale": main_cfg.combine_scale,
                   "active_experts": main_nums["active_experts"], "parallelism": "single GPU"},
        "tflops": round(main_nums["tflops"], 3),
        "gbps": round(main_nums["gbps"], 1),
        "hbm_frac": round(main_nums["hbm_frac"], 4),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prefill_8192": prefill,
        "prefill_8192_all_experts": uniform,
        "fp8_decode_64": fp8_decode,
        "fp8_prefill_8192": fp8_prefill,
        "quantize_32768x5120": quant,
        "stack_4x4096": stack,
        "ceilings": ceil,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
