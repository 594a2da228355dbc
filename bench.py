"""Benchmark of the block-scaled FP8 GEMM + amax on one MI355X.

One step = one full pass of the path over one batch of synthetic input:
clear Amax, then the GEMM kernel (dequantise + contract + C store + amax),
i.e. exactly what mxgemm_amax queues.  Inputs are generated on the host,
copied to HBM before timing, and stay resident.

Default workload: the projection-shaped GEMM+amax, M=8192 tokens,
N=24576 (128 heads x 192), K=1536, L=1, sf_vec_size=32, E4M3 A/B from
MX-quantised N(0,1) (B scaled by 1/sqrt(K)).  --workload selects another.

Prints one JSON line: TFLOP/s of the whole step, the GEMM kernel's own
duration (HIP events on the launch stream around each GEMM launch), its
roofline against the MFMA peak of the datapath it uses, and the CPU oracle
timed on a bounded sample on this host.

    python bench.py [--steps K] [--warmup W] [--workload 1..5] [--fp8-mfma]
"""

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Published MI355X dense matrix peaks (TFLOP/s)
PEAK_BF16 = 2500.0
PEAK_FP8 = 5000.0
SCLK_PEAK_MHZ = 2400.0  # the engine clock the published MFMA peaks are quoted at
HBM_GBS = 8000.0

CSRC = os.path.join(ROOT, "block_scaled_precision_e4m3_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_PROBE_BYTES = 1 << 30   # float32 bytes read (and written) by each calibration copy


def kernel_source_hash():
    """Short digest of the HIP sources; a traffic figure is only valid for the source it was taken on."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def profile_name(workload_name, fp8_mfma, op="gemm"):
    if op == "quantize":
        return f"mx_quantize_kernel__{workload_name}_operands.txt"
    if op == "proj":
        return f"mxgemm_amax_big_kernel_projection_epilogue__{workload_name}_pipeline.txt"
    return f"mxgemm_amax_big_kernel_{'fp8' if fp8_mfma else 'bf16'}__{workload_name}.txt"


def read_traffic(workload_name, fp8_mfma, op="gemm", key="traffic_bytes_per_launch"):
    """HBM bytes per launch from the committed counter summary, or None if absent or taken on other sources."""
    path = os.path.join(PROFILES, profile_name(workload_name, fp8_mfma, op))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^([a-z_0-9]+):\s*(\S+)\s*$", line)
            if m:
                kv[m.group(1)] = m.group(2)
    if kv.get("kernel_source_sha256") != kernel_source_hash() or key not in kv:
        return None
    return int(kv[key])


def sustained_clock(step, seconds=1.5):
    """Median engine clock (MHz) that rocm-smi reports while `step` runs back to back for `seconds`
    (the clock the chip holds under this load; the MFMA peaks are quoted at 2400 MHz), or None."""
    import shutil
    import subprocess
    import threading

    import torch
    smi = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    if not os.path.exists(smi):
        return None
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            r = subprocess.run([smi, "--showclocks", "--json"], capture_output=True, text=True)
            try:
                card = json.loads(r.stdout)
                card = card[sorted(card)[0]]
                for k, v in card.items():
                    if k.startswith("sclk clock speed"):
                        samples.append(int(re.findall(r"(\d+)Mhz", str(v))[0]))
            except (ValueError, KeyError, IndexError):
                pass
            time.sleep(0.1)
    for _ in range(20):  # reach the steady state before sampling
        step()
    torch.cuda.synchronize()
    th = threading.Thread(target=sample)
    th.start()
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    samples = samples[1:] if len(samples) > 2 else samples  # the first may precede the load
    return sorted(samples)[len(samples) // 2] if samples else None


def copy_probe():
    """Three launches of a plain elementwise copy (y = -x, float32) of COPY_PROBE_BYTES: the
    calibration kernel for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = COPY_PROBE_BYTES // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()


def _csv_rows(pattern):
    rows = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _is_gemm(name):
    return "mxgemm_amax" in name and "reset" not in name and not _is_fused_proj(name)


def _is_fused_proj(name):
    # the tile kernel instantiated with the projection epilogue (C type 4, 256x256 tiles), by its
    # demangled or mangled name
    return "mxgemm_amax_big_kernel" in name and (", 4, 256>" in name or ", 4, 256, " in name or "ELi4ELi256E" in name)


def _is_quantize(name):
    return "mx_quantize_kernel" in name


def _is_proj_rope(name):
    return "proj_rope_mxfp8_kernel" in name


# the projection pipeline's shape: the projection workload's GEMM, 128 heads x 192, 64 rotary features
PROJ_HEADS, PROJ_HEAD_DIM, PROJ_QK_ROPE = 128, 192, 64


def proj_rope_bytes(tokens, n, qr):
    """Algorithmic bytes of the RoPE + dual MXFP8 kernel: float32 Y read, bf16 cos and sin read, both
    directions' codes and scale bytes written."""
    return 4 * tokens * n + 2 * 2 * tokens * qr + 2 * tokens * n + 2 * (tokens * n // 32)


def proj_fused_bytes(tokens, n, k, sf):
    """Algorithmic bytes of the fused projection kernel: A and B codes and their atoms read, bf16 cos and sin
    read (64 rotary features), both directions' codes and scale bytes written."""
    import workloads as W
    return (tokens * k + n * k + W.sf_bytes(tokens, k, 1, sf) + W.sf_bytes(n, k, 1, sf) + 2 * 2 * tokens * 64
            + 2 * tokens * n + 2 * (tokens * n // 32))


def quantize_operands_shape(workload):
    """The stacked float32 operands of a GEMM workload, quantised as one (L, M + N, K) tensor.

    A's rows then B's rows: M is a multiple of 128 for the workloads this is used on, so the
    scale atoms of the stack are exactly those of A followed by those of B."""
    import workloads as W
    cfg = W.WORKLOADS[workload]
    assert cfg["M"] % 128 == 0, "stacking needs A's rows to end on an atom boundary"
    return cfg["L"], cfg["M"] + cfg["N"], cfg["K"], cfg["sf"]


def quantize_bytes(mn, k, l, sf):
    """Algorithmic bytes of one MX quantisation: float32 in, one code byte out per element, plus the atoms."""
    import workloads as W
    return 4 * l * mn * k + l * mn * k + W.sf_bytes(mn, k, l, sf)


def _per_dispatch(rows, kernel_substr, counter, kernel_name_exact=False):
    per = {}
    for r in rows:
        name = r["Kernel_Name"]
        hit = name == kernel_substr if kernel_name_exact else kernel_substr in name
        if hit and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(per.values())


def rocprof_summary(d, workload, fp8_mfma, commands, op="gemm"):
    """Text summary of a rocprofv3 kernel trace (d/kt), two counter passes (d/fetch, d/write) and,
    when present, a matrix-core counter pass (d/mfma)."""
    import workloads as W
    cfg = W.WORKLOADS[workload]
    M, N, K, L, sf = cfg["M"], cfg["N"], cfg["K"], cfg["L"], cfg["sf"]
    if op == "quantize":
        ql, qmn, qk, qsf = quantize_operands_shape(workload)
        out = [f"# rocprofv3 summary: the MX quantisation kernel, the float32 operands of workload {cfg['name']} "
               f"stacked as one ({ql}, {qmn}, {qk}) tensor (A's {M} rows, then B's {N}), sf={qsf}, E4M3", ""]
        is_target = _is_quantize
    elif op == "proj":
        out = [f"# rocprofv3 summary: the projection pipeline of workload {cfg['name']} (tokens={M}, "
               f"{PROJ_HEADS} heads x {PROJ_HEAD_DIM}, {PROJ_QK_ROPE} rotary features, K={K}): the GEMM with the "
               f"RoPE + dual-direction MXFP8 epilogue (fused), and the unfused pipeline's RoPE + MXFP8 kernel", ""]
        is_target = _is_fused_proj
    else:
        out = [f"# rocprofv3 summary: the GEMM + amax kernel ({'fp8 MFMA' if fp8_mfma else 'bf16 MFMA'} path), "
               f"workload {cfg['name']} (M={M} N={N} K={K} L={L} sf={sf})", ""]
        is_target = _is_gemm
    out.append("commands (from the repository root; rocprofv3 runs from /tmp with TMPDIR=/tmp):")
    out.extend("  " + c for c in commands)
    out.append("")
    stats = _csv_rows(os.path.join(d, "kt", "**", "*kernel_stats.csv"))
    out.append("kernel trace (--kernel-trace --stats):")
    avg_us = None
    gemm_name, gemm_total = None, -1.0
    for r in stats:
        name = r["Name"]
        out.append(f"  {name[:100]:100s} calls {int(r['Calls']):5d}  avg {float(r['AverageNs']) / 1e3:10.2f} us  "
                   f"min {float(r['MinNs']) / 1e3:10.2f}  max {float(r['MaxNs']) / 1e3:10.2f}  "
                   f"{float(r['Percentage']):5.1f}%")
        # the kernel that ran the workload: the one with the largest total time
        if is_target(name) and float(r["TotalDurationNs"]) > gemm_total:
            gemm_name, gemm_total = name, float(r["TotalDurationNs"])
            avg_us = float(r["AverageNs"]) / 1e3
    out.append("")
    rope_name, rope_us = None, None
    if op == "proj":
        for r in stats:
            if _is_proj_rope(r["Name"]):
                rope_name, rope_us = r["Name"], float(r["AverageNs"]) / 1e3
    if avg_us and op == "proj":
        fl = W.flops(M, N, K, L)
        out.append(f"gemm_kernel: {gemm_name}")
        out.append(f"gemm_avg_duration_us: {avg_us:.2f}")
        out.append(f"gemm_tflops_at_avg_duration: {fl / (avg_us * 1e-6) / 1e12:.1f}")
        if rope_us:
            out.append(f"rope_kernel: {rope_name}")
            out.append(f"rope_avg_duration_us: {rope_us:.2f}")
            out.append(f"rope_algorithmic_GBps_at_avg_duration: "
                       f"{proj_rope_bytes(M, N, PROJ_QK_ROPE) / (rope_us * 1e-6) / 1e9:.1f}")
    elif avg_us and op == "quantize":
        out.append(f"kernel: {gemm_name}")
        out.append(f"avg_duration_us: {avg_us:.2f}")
        out.append(f"algorithmic_GBps_at_avg_duration: "
                   f"{quantize_bytes(qmn, qk, ql, qsf) / (avg_us * 1e-6) / 1e9:.1f}")
    elif avg_us:
        fl = W.flops(M, N, K, L)
        out.append(f"gemm_kernel: {gemm_name}")
        out.append(f"gemm_avg_duration_us: {avg_us:.2f}")
        out.append(f"gemm_tflops_at_avg_duration: {fl / (avg_us * 1e-6) / 1e12:.1f}")
    fetch = _csv_rows(os.path.join(d, "fetch", "**", "*counter_collection.csv"))
    write = _csv_rows(os.path.join(d, "write", "**", "*counter_collection.csv"))
    if fetch and write and gemm_name:
        gf = _per_dispatch(fetch, gemm_name, "FETCH_SIZE", kernel_name_exact=True)
        gw = _per_dispatch(write, gemm_name, "WRITE_SIZE", kernel_name_exact=True)
        cf = _per_dispatch(fetch, "neg", "FETCH_SIZE")
        cw = _per_dispatch(write, "neg", "WRITE_SIZE")
        f_fac = COPY_PROBE_BYTES / (1024.0 * sum(cf) / len(cf))
        w_fac = COPY_PROBE_BYTES / (1024.0 * sum(cw) / len(cw))
        fb = sum(gf) / len(gf) * 1024.0 * f_fac
        wb = sum(gw) / len(gw) * 1024.0 * w_fac
        ab = (quantize_bytes(qmn, qk, ql, qsf) if op == "quantize" else
              proj_fused_bytes(M, N, K, sf) if op == "proj" else W.algorithmic_bytes(M, N, K, L, sf))
        out += ["",
                "HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; KiB per dispatch):",
                f"  kernel FETCH_SIZE per dispatch (KiB, mean of {len(gf)}): {sum(gf) / len(gf):.0f}",
                f"  kernel WRITE_SIZE per dispatch (KiB, mean of {len(gw)}): {sum(gw) / len(gw):.0f}",
                f"  copy probe (y = -x, {COPY_PROBE_BYTES} B read + {COPY_PROBE_BYTES} B written): "
                f"FETCH_SIZE {sum(cf) / len(cf):.0f} KiB, WRITE_SIZE {sum(cw) / len(cw):.0f} KiB",
                f"  calibration factors (true bytes / counter bytes): fetch {f_fac:.4f}, write {w_fac:.4f}",
                f"fetch_bytes_per_launch: {fb:.0f}",
                f"write_bytes_per_launch: {wb:.0f}",
                f"traffic_bytes_per_launch: {fb + wb:.0f}",
                f"algorithmic_bytes_per_launch: {ab}",
                f"traffic_over_algorithmic: {(fb + wb) / ab:.3f}"]
        if op == "proj" and rope_name:
            rf = _per_dispatch(fetch, rope_name, "FETCH_SIZE", kernel_name_exact=True)
            rw = _per_dispatch(write, rope_name, "WRITE_SIZE", kernel_name_exact=True)
            if rf and rw:
                rfb = sum(rf) / len(rf) * 1024.0 * f_fac
                rwb = sum(rw) / len(rw) * 1024.0 * w_fac
                rab = proj_rope_bytes(M, N, PROJ_QK_ROPE)
                out += [f"rope_traffic_bytes_per_launch: {rfb + rwb:.0f}",
                        f"rope_algorithmic_bytes_per_launch: {rab}",
                        f"rope_traffic_over_algorithmic: {(rfb + rwb) / rab:.3f}"]
    mfma = _csv_rows(os.path.join(d, "mfma", "**", "*counter_collection.csv"))
    if mfma and gemm_name:
        # SQ_VALU_MFMA_BUSY_CYCLES sums the matrix-core busy cycles of every SIMD;
        # SQ_BUSY_CYCLES sums the busy cycles of every shader engine (32 engines of
        # 8 CUs, so 32 SIMDs to an engine): their ratio over 32 is the fraction of
        # the kernel's cycles the matrix cores were busy, at whatever clock it held
        insts = _per_dispatch(mfma, gemm_name, "SQ_INSTS_MFMA", kernel_name_exact=True)
        busy = _per_dispatch(mfma, gemm_name, "SQ_VALU_MFMA_BUSY_CYCLES", kernel_name_exact=True)
        sq = _per_dispatch(mfma, gemm_name, "SQ_BUSY_CYCLES", kernel_name_exact=True)
        if insts and busy and sq:
            mi, mb, sb = sum(insts) / len(insts), sum(busy) / len(busy), sum(sq) / len(sq)
            out += ["",
                    "matrix cores (--pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES; per dispatch, "
                    f"mean of {len(busy)}):",
                    f"  SQ_INSTS_MFMA {mi:.0f}  SQ_VALU_MFMA_BUSY_CYCLES {mb:.4g}  SQ_BUSY_CYCLES {sb:.4g}",
                    f"mfma_instructions_per_launch: {mi:.0f}",
                    f"mfma_busy_fraction: {mb / (32.0 * sb):.3f}"]
    out += ["", f"kernel_source_sha256: {kernel_source_hash()}"]
    bench_line = os.path.join(d, "bench.json")
    if os.path.exists(bench_line):
        with open(bench_line) as f:
            out += ["", f"bench.py line of the same run ({commands[0].split('  ')[0] if commands else 'bench.py'}):",
                    f.read().strip()]
    return "\n".join(out) + "\n"


def cpu_baseline(p, target_s=12.0):
    """Time the CPU oracle on sampled rows of the workload; scale to TFLOP/s of the GEMM."""
    import numpy as np

    import oracle
    rng = np.random.default_rng(0)
    args = (p["A"], p["B"], p["SFA"], p["SFB"], p["M"], p["N"], p["K"], p["L"], p["sf"], p["a_fmt"], p["b_fmt"])
    rows = 64
    done_rows = 0
    t_total = 0.0
    while t_total < target_s:
        idx = np.sort(rng.choice(p["M"], min(rows, p["M"]), replace=False))
        t0 = time.perf_counter()
        oracle.gemm_rows(*args, 0, idx)
        t_total += time.perf_counter() - t0
        done_rows += len(idx)
        rows *= 2
    flops = 2.0 * done_rows * p["N"] * p["K"]
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"oracle.gemm_rows (fp64 decode + SF-atom expansion + C and sum|a||b| GEMMs via numpy BLAS) "
                   f"on batch 0 rows drawn in doubling sets of distinct rows (64, 128, ... up to M; a row can recur "
                   f"between sets), {done_rows} rows x {p['N']} x {p['K']} in all, {t_total:.1f} s; "
                   f"value counts the 2*rows*N*K flops of C only"),
    }


def host_overhead(lib, A, B, SFA, SFB, C, Amax, stream_handle, a_fmt, b_fmt, sf, batches=5, calls=200):
    """CPU time of one mxgemm_amax call through the C ABI: validation, the Amax clear and the kernel
    launch, without waiting for the GPU.  A 128x128x128 problem over the workload's own buffers (every
    workload is at least that large), called straight through ctypes with prepared integer arguments;
    the mean over `batches` batches of `calls` calls, the queue drained between batches (untimed)."""
    import torch
    f = lib._lib.mxgemm_amax
    args = (A.data_ptr(), B.data_ptr(), SFA.data_ptr(), SFB.data_ptr(), C.data_ptr(), Amax.data_ptr(),
            128, 128, 128, 1, sf, a_fmt, b_fmt, stream_handle)
    assert f(*args) == lib.MXG_OK
    torch.cuda.synchronize()
    total = 0.0
    for _ in range(batches):
        t0 = time.perf_counter()
        for _ in range(calls):
            f(*args)
        total += time.perf_counter() - t0
        torch.cuda.synchronize()
    # the same through a plan: validation and configuration done once, pointer checks per call
    plan = lib.Plan(128, 128, 128, 1, sf, a_fmt, b_fmt)
    fp = lib._lib.mxgemm_plan_execute
    pargs = (plan._ref,) + args[:6] + (stream_handle,)
    assert fp(*pargs) == lib.MXG_OK
    torch.cuda.synchronize()
    ptotal = 0.0
    for _ in range(batches):
        t0 = time.perf_counter()
        for _ in range(calls):
            fp(*pargs)
        ptotal += time.perf_counter() - t0
        torch.cuda.synchronize()
    # the same plan call captured once into a graph (Amax clear + GEMM) and replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        assert fp(*(pargs[:-1] + (side.cuda_stream,))) == lib.MXG_OK
    torch.cuda.synchronize()
    gtotal = 0.0
    for _ in range(batches):
        t0 = time.perf_counter()
        for _ in range(calls):
            g.replay()
        gtotal += time.perf_counter() - t0
        torch.cuda.synchronize()
    return {"us_per_call": round(total / (batches * calls) * 1e6, 2),
            "plan_us_per_call": round(ptotal / (batches * calls) * 1e6, 2),
            "graph_replay_us": round(gtotal / (batches * calls) * 1e6, 2), "calls": batches * calls,
            "shape": "128x128x128", "what": "mxgemm_amax via ctypes: validate, clear Amax, launch; no wait "
                                            "(plan: mxgemm_plan_execute; graph: one captured plan call, "
                                            "torch CUDAGraph.replay)",
            "pages": "~15 us per launch for the pages' class API with pre-allocated outputs (hardware not stated)"}


def bench_quantize(args):
    """One JSON line for the MX quantisation kernel: a step quantises the workload's float32 A and B,
    stacked as one tensor (see quantize_operands_shape), resident in HBM."""
    import math

    import numpy as np
    import torch

    import block_scaled_precision_e4m3_amd as lib
    import workloads as W
    cfg = W.WORKLOADS[args.workload]
    l, mn, k, sf = quantize_operands_shape(args.workload)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.workload)
    x = torch.randn((l, mn, k), generator=gen, device=dev, dtype=torch.float32)
    if cfg["name"] == "projection":
        x[:, cfg["M"]:, :] /= math.sqrt(k)          # B ~ N(0,1)/sqrt(K), A ~ N(0,1), as in the workload
    q = torch.empty((l, mn, k), dtype=torch.uint8, device=dev)
    sfb = torch.empty(W.sf_bytes(mn, k, l, sf), dtype=torch.uint8, device=dev)
    fmt = lib.MXG_FMT_E4M3
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step():
        lib.mxgemm_mx_quantize(x, q, sfb, mn, k, l, sf, fmt, sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    nbytes = quantize_bytes(mn, k, l, sf)
    ms_per_step = wall * 1e3 / args.steps
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    out = {
        "metric": "MX block quantisation GB/s (float32 in; E4M3 codes and E8M0 scale atoms out)",
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 in, e4m3 codes + e8m0 scales out",
        "data": "synthetic (seeded normal; the workload's operand distributions)",
        "config": {"workload": f"{cfg['name']} operands (A {cfg['M']}x{k} and B {cfg['N']}x{k} stacked)",
                   "MN": mn, "K": k, "L": l, "sf_vec_size": sf, "fmt": "e4m3"},
        "kernel_ms": round(kernel_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_GBS, 4),
                     "traffic": read_traffic(cfg["name"], False, "quantize"),
                     "algorithmic_bytes": nbytes},
    }
    if args.copy_probe:
        copy_probe()
    if not args.no_cpu_baseline:
        import oracle
        xh = x.cpu().numpy()
        rng = np.random.default_rng(0)
        t_total, done = 0.0, 0
        while t_total < 10.0:
            r0 = 128 * int(rng.integers(0, mn // 128))
            t1 = time.perf_counter()
            oracle.mx_quantize(xh[:, r0:r0 + 1024], sf, fmt)
            t_total += time.perf_counter() - t1
            done += xh[:, r0:r0 + 1024].shape[1]
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count()
        out["cpu_baseline"] = {
            "value": quantize_bytes(done, k, l, sf) / t_total / 1e9, "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"oracle.mx_quantize on {done} rows x {k} (blocks of up to 1024 rows at random atom "
                      f"boundaries), {t_total:.1f} s; value counts the same algorithmic bytes per row"}
    print(json.dumps(out), flush=True)


def bench_proj(args):
    """One JSON line for the projection of the projection page at the projection workload's shape.  A
    step takes the page's inputs (E4M3 codes with row-wise E8M0 scales, bf16 cos / sin) to its four
    outputs: both operands' scales repacked into atoms, then the GEMM with the per-head RoPE and
    dual-direction MXFP8 quantisation fused into its epilogue.  The unfused pipeline (GEMM into float32
    Y, then the RoPE + quantisation kernel) is timed beside it, and both give the same bytes."""
    import numpy as np
    import torch

    import block_scaled_precision_e4m3_amd as lib
    import workloads as W
    heads, d, qr = PROJ_HEADS, PROJ_HEAD_DIM, PROJ_QK_ROPE
    p = W.make_workload(5)
    tokens, n, k, sf = p["M"], p["N"], p["K"], p["sf"]
    assert n == heads * d
    kb = W.cdiv(k, sf)

    def rowwise(phys, mn):
        # the (mn, kb) byte of the physical (1, MNb, Kg, 32, 4, 4) atom buffer
        v = phys.reshape(-1, W.cdiv(k, 4 * sf), 32, 4, 4)
        m, b = np.arange(mn)[:, None], np.arange(kb)[None, :]
        return np.ascontiguousarray(v[m // 128, b // 4, m % 32, (m // 32) % 4, b % 4])

    dev = torch.device("cuda:0")
    A, B = torch.from_numpy(p["A"][0]).to(dev), torch.from_numpy(p["B"][0]).to(dev)
    xs = torch.from_numpy(rowwise(p["SFA"], tokens)).to(dev)
    ws = torch.from_numpy(rowwise(p["SFB"], n)).to(dev)
    sfa = torch.empty(W.sf_bytes(tokens, k, 1, sf), dtype=torch.uint8, device=dev)
    sfb = torch.empty(W.sf_bytes(n, k, 1, sf), dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    theta = torch.rand((tokens, qr // 2), generator=gen, device=dev) * 6.283185307179586
    cs = torch.cos(theta).repeat(1, 2).to(torch.bfloat16).contiguous()
    sn = torch.sin(theta).repeat(1, 2).to(torch.bfloat16).contiguous()
    Y = torch.empty((tokens, n), dtype=torch.float32, device=dev)
    amax = torch.zeros(4, dtype=torch.float32, device=dev)
    outs = (torch.empty((tokens, heads, d), dtype=torch.float8_e4m3fn, device=dev),
            torch.empty((tokens, heads, d // 32), dtype=torch.uint8, device=dev),
            torch.empty((tokens, heads, d), dtype=torch.float8_e4m3fn, device=dev),
            torch.empty((tokens // 32, heads, d), dtype=torch.uint8, device=dev))
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    # the fused path: the page's interface (row-wise scales) -> repacks into a workspace -> the GEMM with the
    # RoPE + dual MXFP8 epilogue
    wsp = torch.empty(lib._lib.mxgemm_projection_workspace_bytes(tokens, heads, d, k), dtype=torch.uint8, device=dev)
    fouts = tuple(torch.empty_like(o) for o in outs)

    def step_fused(e=None):
        # what mxgemm_projection_mxfp8 queues (row-wise scale repacks into the workspace, then the fused
        # kernel), called kernel by kernel here so that events can time the fused kernel alone
        if e:
            e[0].record(stream)
        lib.mxgemm_sf_rowwise_to_atoms(xs, sfa, tokens, k, 1, sf, sh)
        lib.mxgemm_sf_rowwise_to_atoms(ws, sfb, n, k, 1, sf, sh)
        if e:
            e[1].record(stream)
        lib.gemm_rope_mxfp8(A, B, sfa, sfb, cs, sn, tokens, heads, d, qr, k, stream=stream, out=fouts)
        if e:
            e[2].record(stream)

    def step(e=None):
        if e:
            e[0].record(stream)
        lib.mxgemm_sf_rowwise_to_atoms(xs, sfa, tokens, k, 1, sf, sh)
        lib.mxgemm_sf_rowwise_to_atoms(ws, sfb, n, k, 1, sf, sh)
        if e:
            e[1].record(stream)
        lib.mxgemm_amax(A, B, sfa, sfb, Y, amax, tokens, n, k, 1, sf, lib.MXG_FMT_E4M3, lib.MXG_FMT_E4M3, sh)
        if e:
            e[2].record(stream)
        lib.proj_rope_mxfp8(Y, cs, sn, heads, d, qr, stream=stream, out=outs)
        if e:
            e[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / args.steps for j in range(3)]
    ms_unfused = wall * 1e3 / args.steps
    for _ in range(args.warmup):
        step_fused()
    torch.cuda.synchronize()
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_fused(fev[i])
    torch.cuda.synchronize()
    wall_f = time.perf_counter() - t0
    fused_repack_ms = sum(e[0].elapsed_time(e[1]) for e in fev) / args.steps
    fused_ms = sum(e[1].elapsed_time(e[2]) for e in fev) / args.steps
    for a, b in zip(outs, fouts):     # the fused outputs equal the unfused pipeline's
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "fused and unfused projections differ"
    # and so do those of the page-interface entry point (workspace, three kernels)
    pouts = lib.projection_mxfp8(A, B, xs, ws, cs, sn, heads, d, qr, workspace=wsp, stream=stream)
    torch.cuda.synchronize()
    for a, b in zip(outs, pouts):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "projection entry point differs"
    ms_per_step = wall_f * 1e3 / args.steps
    flops = W.flops(tokens, n, k, 1)
    rope_bytes = proj_rope_bytes(tokens, n, qr)
    rope_gbs = rope_bytes / (part[2] * 1e-3) / 1e9
    out = {
        "metric": "projection GEMM + RoPE + dual-direction MXFP8 TFLOP/s (GEMM flops over the whole step; "
                  "fused path)",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 codes in, fp32 Y, e4m3 codes + e8m0 scales out",
        "data": "synthetic (seeded, MX-quantised; random rotary angles)",
        "config": {"workload": "projection pipeline", "tokens": tokens, "num_heads": heads, "head_dim": d,
                   "qk_rope": qr, "q_lora": k, "sf_vec_size": sf},
        "repack_ms": round(fused_repack_ms, 4), "fused_kernel_ms": round(fused_ms, 4),
        "unfused": {"ms_per_step": round(ms_unfused, 4), "repack_ms": round(part[0], 4), "gemm_ms": round(part[1], 4),
                    "rope_quant_ms": round(part[2], 4),
                    "what": "row-wise scale repacks, the GEMM into float32 Y, then the RoPE + dual MXFP8 kernel"},
        "roofline": {"kernel": "gemm_rope_mxfp8 (fused)", "bound": "mfma",
                     "achieved": round(flops / (fused_ms * 1e-3) / 1e12, 2), "peak": PEAK_FP8, "unit": "TFLOP/s",
                     "frac": round(flops / (fused_ms * 1e-3) / 1e12 / PEAK_FP8, 4),
                     "peak_of_datapath": PEAK_BF16,
                     "frac_of_datapath_peak": round(flops / (fused_ms * 1e-3) / 1e12 / PEAK_BF16, 4),
                     "traffic": read_traffic(W.WORKLOADS[5]["name"], False, "proj"),
                     "algorithmic_bytes": proj_fused_bytes(tokens, n, k, sf)},
        "unfused_rope_kernel_roofline": {"bound": "hbm", "achieved": round(rope_gbs, 1), "peak": HBM_GBS,
                                         "unit": "GB/s", "frac": round(rope_gbs / HBM_GBS, 4),
                                         "traffic": read_traffic(W.WORKLOADS[5]["name"], False, "proj",
                                                                 "rope_traffic_bytes_per_launch"),
                                         "algorithmic_bytes": rope_bytes},
    }
    if args.copy_probe:
        copy_probe()
    if not args.no_cpu_baseline:
        import oracle
        yh = Y.cpu().numpy()
        ch, shh = cs.float().cpu().numpy(), sn.float().cpu().numpy()
        t_total, done = 0.0, 0
        while t_total < 10.0:
            t1 = time.perf_counter()
            r0 = 256 * ((done // 256) % (tokens // 256))
            oracle.proj_rope_mxfp8(yh[r0:r0 + 256], ch[r0:r0 + 256], shh[r0:r0 + 256], heads, d, qr)
            t_total += time.perf_counter() - t1
            done += 256
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count()
        out["cpu_baseline"] = {
            "value": rope_bytes * done / tokens / t_total / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle.proj_rope_mxfp8 (RoPE + both quantisation directions) on {done} tokens in blocks of "
                      f"256, {t_total:.1f} s; value counts the RoPE kernel's algorithmic bytes per token"}
    print(json.dumps(out), flush=True)


def bench_probe(args):
    """One JSON line of hardware ceilings measured on this GPU (include/mxgemm_probe.h): the dense MFMA
    rate and shader clock with all CUs busy (bf16 32x32x16 and scaled FP8 32x32x64), the global->LDS
    operand path at the GEMM's per-step block counts, and HBM streaming read and write bandwidth."""
    import ctypes

    import numpy as np
    import torch

    import block_scaled_precision_e4m3_amd as lib
    plib = lib._lib
    vp, ci, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
    plib.mxprobe_mfma.argtypes = [ci, ci, ci, vp, vp]
    plib.mxprobe_copy_lds.argtypes = [vp, u64, ci, ci, ci, ci, ctypes.c_uint, vp, vp]
    plib.mxprobe_hbm.argtypes = [ci, vp, u64, ci, vp, vp]
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
        return best

    out = {"metric": "MI355X ceilings measured by probes", "n_gpus": 1, "device": props.name, "cus": cus}
    spans = torch.zeros(2 * cus, dtype=torch.int64, device=dev)
    for kind, name, fl in ((0, "bf16_32x32x16", 32768), (1, "fp8_scaled_32x32x64", 131072)):
        iters = 20000 if kind == 0 else 10000
        t = timed(lambda: plib.mxprobe_mfma(kind, cus, iters, spans.data_ptr(), sh))
        sp = spans.view(cus, 2).cpu().numpy().astype(np.float64)
        clk = float(np.mean(sp[:, 0] / sp[:, 1])) * 100e6
        flops = 4.0 * cus * iters * 8 * fl
        out[f"mfma_{name}"] = {"tflops": round(flops / t / 1e12, 1), "sclk_ghz": round(clk / 1e9, 3),
                               "tflops_per_ghz": round(flops / t / 1e12 / (clk / 1e9), 1),
                               "what": f"{cus} workgroups x 4 waves x {iters} x 8 independent MFMAs"}
    region = 2 << 20
    src = torch.randint(0, 255, (32 << 20,), dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    steps = 2000
    for per_step, vgpr, stride in ((16, 0, 0), (16, 1, 0), (8, 0, 0), (16, 0, 1536), (16, 0, 2048), (16, 0, 4096),
                                   (16, 0, 2176), (8, 0, 2048)):
        reg = region if stride == 0 else max(region, 64 * 8 * stride)
        t = timed(lambda: plib.mxprobe_copy_lds(src.data_ptr(), reg, cus, steps, per_step, vgpr, stride,
                                                 sink.data_ptr(), sh))
        nbytes = float(cus) * steps * 4 * per_step * 1024
        key = f"l2_to_{'vgpr' if vgpr else 'lds'}_{per_step}KB_per_wave_step" + (f"_rows_at_{stride}" if stride else "")
        out[key] = {"GBps": round(nbytes / t / 1e9, 1), "per_cu_bytes_per_ns": round(nbytes / t / 1e9 / cus, 2),
                    "us_per_step": round(t / steps * 1e6, 3),
                    "what": f"{cus} workgroups x 4 waves, {per_step} x 1 KB per wave per step "
                            f"({'contiguous' if not stride else f'8 rows x 128 B, {stride} B apart'}) from a "
                            f"{reg >> 20} MB region, wait + barrier per step, {steps} steps"}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    for write in (1, 0):
        t = timed(lambda: plib.mxprobe_hbm(write, buf.data_ptr(), nbytes, 8 * cus, sink.data_ptr(), sh))
        out["hbm_write" if write else "hbm_read"] = {"GBps": round(nbytes / t / 1e9, 1),
                                                     "frac_of_8TBps": round(nbytes / t / 8e12, 3),
                                                     "what": f"{nbytes >> 30} GiB, 16-byte accesses, "
                                                             f"{8 * cus} workgroups x 256 threads"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--op", choices=["gemm", "quantize", "proj", "probe"], default="gemm",
                    help="gemm: the GEMM + amax step (default); quantize: the MX quantisation of the "
                         "workload's float32 operands; proj: the projection pipeline (row-wise scales -> GEMM -> "
                         "RoPE + dual-direction MXFP8) at the projection workload's shape; probe: hardware "
                         "ceilings (MFMA rate and clock, global->LDS path, HBM bandwidth)")
    ap.add_argument("--fp8-mfma", action="store_true", help="time the reduced-precision FP8 MFMA path")
    ap.add_argument("--fp4", action="store_true",
                    help="the workload's shape with packed FP4 (E2M1) operands and sf = 32 (same value recipe)")
    ap.add_argument("--sf-rowwise", action="store_true",
                    help="scales arrive row-wise (rows, ceil(K/sf)) bytes, as on the projection page's MXFP8 "
                         "input path; a step repacks both into the atom layout, then runs the GEMM")
    ap.add_argument("--c-dtype", choices=["f32", "bf16", "f16"], default="f32",
                    help="C element type (f32, the default, is the operation's own output)")
    ap.add_argument("--c-major", choices=["n", "m"], default="n",
                    help="C layout: n-major (L, M, N), the default, or m-major (L, N, M) (float32 C)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-host-overhead", action="store_true",
                    help="skip the 1000 small calls that time the host side (keeps profiles to the workload)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the sustained-clock reading (1.5 s of back-to-back steps under rocm-smi)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, run the copy kernel that calibrates the HBM byte counters")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="no GPU work: summarise rocprofv3 output under DIR (kt/, fetch/, write/) and print it")
    ap.add_argument("--command", action="append", default=[],
                    help="with --rocprof-summary: a command line to record in the summary (repeatable)")
    args = ap.parse_args()

    if args.rocprof_summary:
        print(rocprof_summary(args.rocprof_summary, args.workload, args.fp8_mfma, args.command, args.op), end="")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only (--gpus 1); several GPUs would each run this kernel "
              "on their own share of C tiles, which this benchmark does not launch", file=sys.stderr)
        sys.exit(2)

    if args.op == "quantize":
        bench_quantize(args)
        return
    if args.op == "proj":
        bench_proj(args)
        return
    if args.op == "probe":
        bench_probe(args)
        return

    import torch

    import block_scaled_precision_e4m3_amd as lib
    import workloads as W

    if args.fp4:
        cfg = W.WORKLOADS[args.workload]
        p = W.make_problem(cfg["M"], cfg["N"], cfg["K"], cfg["L"], 32, W.FMT_E2M1, W.FMT_E2M1, seed=args.workload,
                           b_scale=float(1.0 / math.sqrt(cfg["K"])) if cfg["name"] == "projection" else 1.0)
    else:
        p = W.make_workload(args.workload)
    M, N, K, L, sf = p["M"], p["N"], p["K"], p["L"], p["sf"]
    dev = torch.device("cuda:0")
    A = torch.from_numpy(p["A"]).to(dev)
    B = torch.from_numpy(p["B"]).to(dev)
    SFA = torch.from_numpy(p["SFA"]).to(dev)
    SFB = torch.from_numpy(p["SFB"]).to(dev)
    C = torch.empty(L * M * N, dtype=torch.float32, device=dev)
    Amax = torch.zeros(4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    mode_flag = (lib.MXG_FLAG_FP8_MFMA if args.fp8_mfma else 0) | \
        {"f32": 0, "bf16": lib.MXG_FLAG_C_BF16, "f16": lib.MXG_FLAG_C_F16}[args.c_dtype] | \
        (lib.MXG_FLAG_C_MMAJOR if args.c_major == "m" else 0)

    if args.sf_rowwise:
        import numpy as np
        kb = W.cdiv(K, sf)
        # the workload's scales, re-expressed row-wise: byte (l, row, kb) of the atom layout
        def rowwise_of(phys, mn):
            mnb, kg = W.cdiv(mn, 128), W.cdiv(K, 4 * sf)
            v = np.asarray(phys).reshape(L, mnb, kg, 32, 4, 4).transpose(0, 1, 4, 3, 2, 5)
            return np.ascontiguousarray(v.reshape(L, mnb * 128, kg * 4)[:, :mn, :kb])
        RA = torch.from_numpy(rowwise_of(p["SFA"], M)).to(dev)
        RB = torch.from_numpy(rowwise_of(p["SFB"], N)).to(dev)

    def repack():
        lib.mxgemm_sf_rowwise_to_atoms(RA, SFA, M, K, L, sf, sh)
        lib.mxgemm_sf_rowwise_to_atoms(RB, SFB, N, K, L, sf, sh)

    def step():
        if args.sf_rowwise:
            repack()
        lib.mxgemm_amax_ex(A, B, SFA, SFB, C, Amax, M, N, K, L, sf, p["a_fmt"], p["b_fmt"], mode_flag, sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    rp_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        # one step == mxgemm_amax: the Amax-clearing kernel, then the GEMM kernel (after the
        # scale repacks when the scales arrive row-wise)
        if args.sf_rowwise:
            rp_ev[i][0].record(stream)
            repack()
            rp_ev[i][1].record(stream)
        lib.mxgemm_amax_reset(Amax, sh)
        ev[i][0].record(stream)
        lib.mxgemm_amax_ex(A, B, SFA, SFB, C, Amax, M, N, K, L, sf, p["a_fmt"], p["b_fmt"],
                           mode_flag | lib.MXG_FLAG_AMAX_ACCUMULATE, sh)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps

    flops = W.flops(M, N, K, L)
    ms_per_step = wall * 1e3 / args.steps
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    # the metric's peak: MI355X dense MXFP8 MFMA; the default datapath contracts on the bf16
    # MFMA, whose own peak is half that (its fraction is reported beside)
    peak = PEAK_FP8
    tile_m, tile_n, grid = lib.mxgemm_launch_config(M, N, K, L, sf)
    abytes = W.algorithmic_bytes(M, N, K, L, sf)

    out = {
        "metric": "block-scaled FP8 GEMM+amax TFLOP/s and % of MI355X MXFP8 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp4-e2m1 codes, exact bf16 dequant, fp32 accumulate" if args.fp4 else
                  "fp8-e4m3 codes, exact bf16 dequant, fp32 accumulate" if not args.fp8_mfma
                  else "fp8-e4m3 scaled MFMA (reduced-precision sums), fp32 accumulate"),
        "data": "synthetic (seeded, MX-quantised)",
        "config": {"workload": W.WORKLOADS[args.workload]["name"], "M": M, "N": N, "K": K, "L": L,
                   "sf_vec_size": sf, "a_fmt": ["e4m3", "e5m2", "e2m1"][p["a_fmt"]],
                   "b_fmt": ["e4m3", "e5m2", "e2m1"][p["b_fmt"]], "tile": f"{tile_m}x{tile_n}", "grid": grid,
                   "path": "fp8-mfma" if args.fp8_mfma else "bf16-mfma", "c_dtype": args.c_dtype,
                   "c_major": args.c_major,
                   "sf_layout": "row-wise, repacked each step" if args.sf_rowwise else "atoms"},
        "pct_of_mxfp8_peak": round(100.0 * achieved / PEAK_FP8, 2),
        "kernel_ms": round(kernel_ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "peak_of_datapath": PEAK_FP8 if args.fp8_mfma else PEAK_BF16,
                     "frac_of_datapath_peak": round(achieved / (PEAK_FP8 if args.fp8_mfma else PEAK_BF16), 4),
                     "traffic": read_traffic(W.WORKLOADS[args.workload]["name"], args.fp8_mfma),
                     "algorithmic_bytes": abytes,
                     "algorithmic_GBps": round(abytes / (kernel_ms * 1e-3) / 1e9, 1)},
    }
    if args.sf_rowwise:
        out["repack_ms"] = round(sum(a.elapsed_time(b) for a, b in rp_ev) / args.steps, 4)
    if not args.no_clock:
        mhz = sustained_clock(step)
        if mhz:
            dp = PEAK_FP8 if args.fp8_mfma else PEAK_BF16
            out["clock"] = {"sclk_mhz_sustained": mhz, "sclk_mhz_of_peaks": SCLK_PEAK_MHZ,
                            "datapath_peak_at_sustained_clock": round(dp * mhz / SCLK_PEAK_MHZ, 1),
                            "frac_of_datapath_peak_at_sustained_clock": round(achieved / (dp * mhz / SCLK_PEAK_MHZ), 4),
                            "what": "engine clock rocm-smi reports while the step runs back to back for 1.5 s"}
    if not args.no_host_overhead:
        out["host_overhead"] = host_overhead(lib, A, B, SFA, SFB, C, Amax, sh, p["a_fmt"], p["b_fmt"], sf)
    if args.copy_probe:
        copy_probe()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
