"""Benchmark of the SPECTRE spectral mix forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

A step is one spectre_mix_fwd call over the whole workload (all passes of
the hot path: forward transforms of q, k, v, the gated spectral product, the
inverse transform, residual + LayerNorm), with every input already resident
in device memory.  W untimed steps, then exactly K timed steps between two
device synchronisations.  Prints one JSON line:

  value        tokens/s = B * L * K / (timed seconds), one GPU
  roofline     the dominant kernel's algorithmic bytes per launch divided by
               its average duration (HIP events recorded by the library on
               its own stream over K traced calls), against 8 TB/s HBM;
               `traffic` is HBM bytes per launch from the committed
               rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled by a plain
               copy's reading), or null when the kernels have changed since
  whole_call   the byte model of the whole call and its fraction of 8 TB/s;
               also the median of up to 50 calls timed one at a time with
               the 256 MB memory-side cache cleared before each (a 1 GiB
               fill outside the events): flushed_ms_median
  cpu_baseline the CPU oracle timed on this host on the whole workload, on
               the host threads this job is given (OMP_NUM_THREADS when
               set, else every online CPU), with the CPU model named

The default workload is the article's long-context shape B=1, L=65536, H=8,
D=64 in binary32 with no truncation.

Other modes (used to produce the files under profiles/):
    --profile-run        the timed steps only (no CPU baseline), plus one
                         known-size device copy for counter calibration
    --summarize DIR ...  turn rocprofv3 output directories into the text
                         summaries kept under profiles/
    --write-counters FETCH_DIR WRITE_DIR
                         write profiles/hbm_counters.json from a FETCH_SIZE
                         and a WRITE_SIZE run of --profile-run
"""
from __future__ import annotations

import argparse
import dataclasses
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
CSRC = os.path.join(ROOT, "efficient_attention_fft_amd", "csrc")
COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written
FLUSH_BYTES = 1 << 30  # fill that clears the 256 MB memory-side cache before a flushed call


def source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def kernel_bytes(name: str, w, gate_kind: int = 0, local: bool = False,
                 norm_order: int = 0) -> int:
    """Algorithmic HBM bytes of one launch of a pass: every tensor element the
    pass must read or write once (inputs, the spectra it exchanges, outputs,
    the kept gate bins).  A complex gate has 8 bytes per bin, so its gate and
    gate-table bytes double.  With the local branch the pass that normalises
    also reads y_loc (4 bytes per element).  The single-pass column kernel
    (L = 3072, 4096) of a post-norm call without the local branch reads x and
    stores x + y, so its norm pass reads that one tensor."""
    N = w.N
    s = w.elem_bytes
    spec = 4 * N  # one tensor's spectrum as binary32 complex channel pairs
    gb = 8 if gate_kind == 2 else 4  # bytes per gate value
    gate = gb * w.H * min(w.keep_bins, w.nbins)
    if name == "A1_fwd_strided":
        import efficient_attention_fft_amd as sm
        _, (l1, l2, l3) = sm.spectre_mix_plan(w.L)
        folded = 0
        if l3 in (256, 1024):  # multi-level square B kernel: this launch also builds the gate table
            folded = gate + gb * w.H * w.L
        return 3 * N * s + 3 * spec + folded
    if name == "A2_fwd_strided":
        return 6 * spec
    if name == "B_mid_lds":
        import efficient_attention_fft_amd as sm
        _, (l1, l2, l3) = sm.spectre_mix_plan(w.L)
        if l1 == 1 and l2 == 1:  # single level: the kept gate bins themselves
            return 3 * N * s + spec + gate
        if l3 in (256, 1024):
            gate = gb * w.H * w.L  # the gate table A1's launch writes
        return 3 * spec + spec + gate
    fold = (norm_order & 1) == 0 and not local
    if name == "B_col":  # q, k, v read once, the kept gate bins, y (or x + y) written
        return 3 * N * s + gate + spec + (N * s if fold else 0)
    if name == "C2_inv_strided":
        return 2 * spec
    yl = 4 * N if local else 0
    if name == "C1_inv_norm":
        return spec + 2 * N * s + 8 * w.C + yl
    if name == "C1_inv":
        return 2 * spec
    if name == "LN_norm":
        if fold and w.L in (3072, 4096):  # x + y from the column kernel
            return spec + N * s + 8 * w.C
        return spec + 2 * N * s + 8 * w.C + yl
    if name == "L_local":  # q, k, v read once; y_loc (binary32) written
        return 3 * N * s + 4 * N
    raise KeyError(name)


def model_bytes(w) -> int:
    """The frozen byte model of the whole call: read q, k, v, x once and write
    out once, plus the four-step's exchanges (2 x 4N per forward spectrum and
    2 x 4N for the inverse) when the column does not fit one workgroup."""
    N, s = w.N, w.elem_bytes
    m_min = 5 * N * s + 4 * w.H * min(w.keep_bins, w.nbins) + 8 * w.C
    if w.L <= 4096:
        return m_min
    extra = 32 * N
    if w.L > 65536 * 4:
        extra += 24 * N
    return m_min + extra


def host_threads():
    """Host threads the CPU leg may use: the CPU share this process is
    given (the job's thread allotment, OMP_NUM_THREADS when the environment
    sets one, which a GPU host shares among its GPUs), else every online
    CPU."""
    online = os.cpu_count() or 1
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    return max(1, min(share, online) if share > 0 else online)


def host_cpu():
    """The host CPU's model name and its online CPU count."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return name, os.cpu_count() or 1


def _cpu_fields(threads):
    name, online = host_cpu()
    return {"cores": threads, "cpu_model": name, "cpus_online": online}


def cpu_baseline(w, inp, gate_kind=0, norm_order=0):
    import oracle
    threads = host_threads()
    t0 = time.perf_counter()
    oracle.spectre_mix(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"], inp["gamma"],
                       inp["beta"], w.keep_bins, dtype=w.dtype, nthreads=threads,
                       gate_kind=gate_kind, norm_order=norm_order)
    dt = time.perf_counter() - t0
    return {"value": w.tokens / dt, "unit": "tokens/s", **_cpu_fields(oracle.threads(threads)),
            "kind": "oracle", "sample": "the whole workload once: %d columns x %d tokens, "
            "float64, %.2f s wall" % (w.B * w.C, w.L, dt)}


def cpu_baseline_chunked(w, inp, gate_blocks, F, keep_blk, keep_axis):
    import oracle
    threads = host_threads()
    t0 = time.perf_counter()
    oracle.spectre_mix_chunked(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"], gate_blocks,
                               inp["gamma"], inp["beta"], F, keep_blk, keep_axis, dtype=w.dtype,
                               nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": w.tokens / dt, "unit": "tokens/s", **_cpu_fields(oracle.threads(threads)),
            "kind": "oracle", "sample": "the whole workload once, chunked (fft_len %d): %d "
            "columns x %d tokens, float64, %.2f s wall" % (F, w.B * w.C, w.L, dt)}


def cpu_baseline_local(w, inp, wl, wr, gate_kind=0, norm_order=0):
    import oracle
    threads = host_threads()
    t0 = time.perf_counter()
    oracle.spectre_mix_local(inp["q"], inp["k"], inp["v"], inp["x"], inp["gate"], inp["gamma"],
                             inp["beta"], w.keep_bins, wl, wr, dtype=w.dtype, nthreads=threads,
                             gate_kind=gate_kind, norm_order=norm_order)
    dt = time.perf_counter() - t0
    return {"value": w.tokens / dt, "unit": "tokens/s", **_cpu_fields(oracle.threads(threads)),
            "kind": "oracle", "sample": "the whole workload once with the local branch (keys "
            "t-%d..t+%d): %d columns x %d tokens, float64, %.2f s wall"
            % (wl, wr, w.B * w.C, w.L, dt)}


def traffic_for(kernel: str, w):
    """HBM bytes per launch of `kernel` from the committed counters, or None."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_hash") != source_hash() or c.get("workload") != w.name:
        return None
    k = c.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


def run_bench(args):
    import numpy as np  # noqa: F401
    import torch

    import efficient_attention_fft_amd as sm
    import workloads

    w = workloads.WORKLOADS[args.workload]
    print("bench: workload %s, generating inputs" % w.name, file=sys.stderr, flush=True)
    inp = workloads.make_inputs(w)
    gk, no = args.gate_kind, args.norm_order
    if gk != 0:
        inp["gate"] = workloads.make_gate(w, gk)
    F = args.fft_len
    if F:  # chunked mix: blocks of F tokens, every bin kept in both steps
        inp["gate"], gate_blocks = workloads.make_chunk_gates(w, F)
        keep_blk, keep_axis = F // 2 + 1, (w.L // F) // 2 + 1

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda()
        return torch.from_numpy(a).cuda()

    q, k, v, x = (dev(inp[n]) for n in "qkvx")
    gate, gamma, beta = dev(inp["gate"]), dev(inp["gamma"]), dev(inp["beta"])
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    if F:
        gbd = dev(gate_blocks)

    win = args.window
    wl = wr = win // 2

    def step():
        if win:
            return sm.spectre_mix_fwd_local_ex(q, k, v, x, gate, gamma, beta, out, w.B, w.H, w.L,
                                               w.D, w.keep_bins, wl, wr, w.dtype, gk, no, stream)
        if F:
            return sm.spectre_mix_fwd_chunked(q, k, v, x, gate, gbd, gamma, beta, out, w.B, w.H,
                                              w.L, w.D, F, keep_blk, keep_axis, w.dtype, stream)
        if gk == 0 and no == 0:
            return sm.spectre_mix_fwd(q, k, v, x, gate, gamma, beta, out, w.B, w.H, w.L, w.D,
                                      w.keep_bins, w.dtype, stream)
        return sm.spectre_mix_fwd_ex(q, k, v, x, gate, gamma, beta, out, w.B, w.H, w.L, w.D,
                                     w.keep_bins, w.dtype, gk, no, stream)

    for _ in range(args.warmup):
        sm.check(step())
    torch.cuda.synchronize()
    print("bench: warmup done, timing %d steps" % args.steps, file=sys.stderr, flush=True)

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        sm.check(step())
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = w.tokens * args.steps / wall

    # each call alone with the memory-side cache cleared first: a 1 GiB fill
    # (outside the events) before every call, so no input or workspace line
    # is left in the 256 MB cache from the previous call
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    fl = []
    for _ in range(min(args.steps, 50)):
        flush.zero_()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sm.check(step())
        e1.record(stream)
        e1.synchronize()
        fl.append(e0.elapsed_time(e1))
    del flush
    flushed_ms = float(sorted(fl)[len(fl) // 2])

    # per-kernel durations: the same K calls again, with the library's events
    sm.check(sm.spectre_mix_trace_start(args.steps))
    for _ in range(args.steps):
        sm.check(step())
    st, kernels, ncalls = sm.spectre_mix_trace_stop()
    sm.check(st)
    # per call, summed over a kernel's launches (a pass may run in chunks)
    per_kernel, launches = {}, {}
    for name, tot in kernels:
        per_kernel[name] = per_kernel.get(name, 0.0) + tot / max(ncalls, 1)
        launches[name] = launches.get(name, 0) + 1
    print("bench: per-kernel ms " + json.dumps({k: round(v, 4) for k, v in per_kernel.items()}),
          file=sys.stderr, flush=True)
    dom = max(per_kernel, key=per_kernel.get)
    nl = launches[dom]
    # the chunked mix transforms blocks of F tokens: the passes follow that plan
    wk = w if not F else dataclasses.replace(w, B=w.B * (w.L // F), L=F, keep_bins=F // 2 + 1)
    dom_bytes = kernel_bytes(dom, wk, gk, local=bool(win), norm_order=no) / nl  # per launch
    avg_ms = per_kernel[dom] / nl
    achieved = dom_bytes / (avg_ms * 1e-3) / 1e9
    traffic = traffic_for(dom, w) if gk == 0 and no == 0 and not F and not win else None
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes": int(dom_bytes),
                "avg_ms": round(avg_ms, 5), "launches_per_call": nl}
    mb = model_bytes(w)
    if win:  # the branch reads q, k, v again and sends y_loc through HBM once
        mb += 3 * w.N * w.elem_bytes + 8 * w.N
    whole = {"model_bytes": mb,
             "model_GBps": round(mb / (ms_per_step * 1e-3) / 1e9, 1),
             "model_frac": round(mb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "flushed_ms_median": round(flushed_ms, 5),
             "flushed_model_frac": round(mb / (flushed_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "per_kernel_ms": {k: round(v, 5) for k, v in per_kernel.items()}}

    if args.profile_run:
        # one known-size copy, for scaling the HBM counters
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        src.fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    res = {
        "metric": "tokens/s + achieved HBM GB/s (% peak), FFT spectral mix fwd L=64K H=8 D=64 fp32",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == workloads.F32 else "bf16",
        "data": "synthetic",
        "config": dict(w.describe(), parallelism="single GPU",
                       **({"gate_kind": ["real", "logit", "complex"][gk],
                           "norm": ["post", "pre", "post_rms", "pre_rms"][no]} if (gk or no) else {}),
                       **({"fft_len": F} if F else {}),
                       **({"local_window": [wl, wr]} if win else {})),
        "roofline": roofline,
        "whole_call": whole,
    }
    if not args.profile_run and not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        if win:
            res["cpu_baseline"] = cpu_baseline_local(w, inp, wl, wr, gk, no)
        elif F:
            res["cpu_baseline"] = cpu_baseline_chunked(w, inp, gate_blocks, F, keep_blk, keep_axis)
        else:
            res["cpu_baseline"] = cpu_baseline(w, inp, gk, no)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


# ------------------------------------------------------- rocprofv3 summaries

def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    """Pass name of a library kernel from its demangled name (template
    arguments: k_strided<R, IN, TW, SIGN>, k_strided_split<R, IN, TW>,
    k_final<R, DT, FUSE>); other kernels keep their own name."""
    import re
    if "spectre::k_mid_dma" in name:
        return "B_mid_lds"
    m = re.search(r"spectre::(k_\w+)<([^>]*)>", name)
    if not m:
        return "copy (calibration)" if "copyBuffer" in name else name[:60]
    kern, args = m.group(1), [a.strip() for a in m.group(2).split(",")]
    if kern in ("k_strided", "k_strided_split"):
        return {"1": "A1_fwd_strided", "2": "A2_fwd_strided", "3": "C2_inv_strided"}.get(
            args[2], name[:60])
    if kern == "k_final_split":
        return "C1_inv_norm"
    if kern.startswith("k_mid"):
        return "B_mid_lds"
    if kern == "k_final":
        return "C1_inv_norm" if args[2] == "true" else "C1_inv"
    if kern == "k_col":
        return "B_col"
    if kern in ("k_layernorm", "k_layernorm2"):
        return "LN_norm"
    if kern == "k_local_attn":
        return "L_local"
    return name[:60]


def summarize(dirs, out_json=None):
    """Kernel durations (kernel_stats) and FETCH_SIZE / WRITE_SIZE
    (counter_collection) from rocprofv3 output directories."""
    stats, counters = {}, {}
    for d in dirs:
        for p in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
            for r in _read_csv(p):
                nm = r.get("Name") or r.get("KernelName") or ""
                stats[nm] = r
        for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in _read_csv(p):
                nm = r.get("Kernel_Name") or r.get("Kernel-Name") or r.get("KernelName") or ""
                cn = r.get("Counter_Name") or r.get("Counter-Name") or ""
                val = float(r.get("Counter_Value") or r.get("Counter-Value") or 0)
                key = (nm, cn)
                counters.setdefault(key, []).append(val)
    lines = []
    if stats:
        lines.append("kernel | calls | avg us | min us | max us | total %")
        for nm, r in sorted(stats.items(), key=lambda kv: -float(kv[1].get("TotalDurationNs", 0))):
            avg = float(r.get("AverageNs", 0)) / 1e3
            lines.append("%s | %s | %.2f | %.2f | %.2f | %s" % (
                _short(nm), r.get("Calls"), avg, float(r.get("MinNs", 0)) / 1e3,
                float(r.get("MaxNs", 0)) / 1e3, r.get("Percentage")))
    if counters:
        lines.append("")
        lines.append("kernel | counter | mean per dispatch (KiB) | dispatches")
        for (nm, cn), vals in sorted(counters.items()):
            lines.append("%s | %s | %.1f | %d" % (_short(nm), cn, sum(vals) / len(vals), len(vals)))
    return "\n".join(lines), stats, counters


def write_counters(fetch_dir, write_dir, workload_id):
    """profiles/hbm_counters.json from one FETCH_SIZE and one WRITE_SIZE
    rocprofv3 --pmc run of `bench.py --profile-run`: per kernel, the mean KiB
    per dispatch of each counter times the factor that maps the calibration
    copy's reading onto its known size (1 GiB read, 1 GiB written)."""
    import workloads
    w = workloads.WORKLOADS[workload_id]
    _, _, fc = summarize([fetch_dir])
    _, _, wc = summarize([write_dir])

    def per_kernel(counters, cname):
        out, copy = {}, None
        for (nm, cn), vals in counters.items():
            if cn != cname:
                continue
            kib = sum(vals) / len(vals)
            if "copyBuffer" in nm:
                big = max(vals)  # the 1 GiB copy is the largest copyBuffer dispatch
                copy = big if copy is None else max(copy, big)
            elif "spectre::" in nm:
                out[_short(nm)] = kib
        return out, copy

    fetch, fcopy = per_kernel(fc, "FETCH_SIZE")
    write, wcopy = per_kernel(wc, "WRITE_SIZE")
    if not fcopy or not wcopy:
        raise SystemExit("no calibration copy found in the counter runs")
    ff = COPY_BYTES / (fcopy * 1024.0)
    wf = COPY_BYTES / (wcopy * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        rd = fetch.get(k, 0.0) * 1024.0 * ff
        wr = write.get(k, 0.0) * 1024.0 * wf
        kernels[k] = {"fetch_kib": round(fetch.get(k, 0.0), 1), "write_kib": round(write.get(k, 0.0), 1),
                      "read_bytes": int(rd), "write_bytes": int(wr),
                      "hbm_bytes_per_launch": int(rd + wr),
                      "algorithmic_bytes": kernel_bytes(k, w)}
    doc = {"workload": w.name, "source_hash": source_hash(),
           "copy_calibration": {"bytes_each_way": COPY_BYTES, "fetch_kib": fcopy, "write_kib": wcopy,
                                "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "kernels": kernels}
    with open(COUNTERS, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    return doc


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gate-kind", type=int, default=0, choices=[0, 1, 2],
                    help="0 real gate, 1 logit gate (sigmoid in the kernels), 2 complex gate")
    ap.add_argument("--norm-order", type=int, default=0, choices=[0, 1, 2, 3],
                    help="0 out = LN(x + y), 1 out = x + LN(y); 2, 3: the same with RMSNorm")
    ap.add_argument("--fft-len", type=int, default=0,
                    help="chunked mix with blocks of this many tokens (0: one block, the plain mix)")
    ap.add_argument("--window", type=int, default=0,
                    help="add the local branch: keys t - W/2 .. t + W/2 (0: no local branch)")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--summarize", nargs="+", metavar="DIR")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.write_counters:
        print(json.dumps(write_counters(*args.write_counters, args.workload), indent=1))
        return 0
    if args.summarize:
        text, _, _ = summarize(args.summarize)
        print(text)
        return 0
    if args.window and (args.window % 2 or args.fft_len):
        print("--window takes an even W and no --fft-len", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested; run with --gpus 1)" % args.gpus, file=sys.stderr)
        return 2
    run_bench(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
