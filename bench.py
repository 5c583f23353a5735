"""Benchmark of the exact-attention hot path on one MI355X.

One step is one pass of the whole path on resident synthetic inputs:
  * prefill: attn_fwd on the LFM2-2.6B-shaped GQA workload (B=4, Hq=32,
    Hkv=8, S=4096, D=64, causal, RoPE base 10000, bf16) — RoPE table, key
    rotation and the fused attention kernel;
  * decode: attn_decode_splitkv on the split-KV workload (B=16, Hq=32, Hkv=8,
    D=128, bf16 cache of 32768 positions, lengths U[1024, 32768]) — split
    pass and LSE merge — at the split count that measured fastest among
    4, 8, 16, 32, 64 before the timed region.

Printed: one JSON line.  The timed region runs the K steps' work as K
prefill calls back to back, then K decode calls, with a HIP event at each of
the three boundaries only: every event recorded between two kernels costs
the GPU a few microseconds of idle time (a kernel trace shows ~4 us per
event on MI355X, ~5 us with the default system-scope fence), so no event
sits inside either run.  `value` is the prefill throughput in TFLOP/s
(algorithmic flops 4*B*Hq*S*S*D/2 over the mean attn_fwd call of the timed
prefill run: key rotation + attention kernel); the decode KV-read bandwidth
(median of 50 calls, each after a 512 MiB read flush) and both fractions of
peak sit beside it.  The `roofline` object is for the dominant kernel, the
fused RoPE attention kernel of the headline call, timed by the HIP event
pair that the library attaches to that kernel's dispatch
(attn_profile_begin/_end).  bench.py's own events are created without the
system-scope fence (hipEventDisableSystemFence), which only timing needs.

Modes for rocprofv3 runs (each launches one thing only): --profile-kernel
REPS [--profile-workload NAME] (production attn_fwd calls on a prefill
workload, then a calibration copy), --profile-decode REPS [--profile-splits
N], --profile-backward REPS; and the summary writers --traffic-summary and
--counters-summary.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import exact_attention_28_amd as xa  # noqa: E402
import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
METRIC = "attention fwd TFLOP/s + decode KV GB/s, as % of MI355X MFMA/HBM peak"
KERNEL_SOURCES = ("fwd16p_kernel.h", "common.h", "lds.h")
# the attention kernel of the headline LFM2 prefill call: the software-pipelined
# kernel of unmasked, unsplit launches (template arguments: element type, head
# dim, query heads per workgroup, causal, fused query RoPE, query blocks per wave)
KERNEL_NAME = "fwdp_kernel"
KERNEL_LABEL = "fwdp_kernel<__bf16, D=64, HPW=4, CAUSAL=1, ROPE=1, NQB=2, KS=1, ONEBUF=0>"
KERNEL_LABEL_NOROPE = "fwdp_kernel<__bf16, D=64, HPW=4, CAUSAL=1, ROPE=0, NQB=2, KS=1, ONEBUF=0>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwdp_lfm2_gqa_prefill_s4096_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash():
    """Hash of the prefill kernel's sources with comments and whitespace
    removed, so that a counter summary stays valid across comment edits and
    goes stale when the code changes."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_28_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)  # block comments
        src = re.sub(r"//[^\n]*", " ", src)                # line comments
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(launch_flops_bytes):
    """HBM traffic per launch of the prefill kernel from the committed
    rocprofv3 counter summary, or None when the kernel changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for ln in open(TRAFFIC_FILE):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed(fn, reps, stream, between=None):
    """Median duration (ms) of fn() over reps, each bracketed by HIP events on
    stream; `between` (e.g. a cache flush) runs before each repetition,
    outside the events."""
    starts = [HipEvent() for _ in range(reps)]
    ends = [HipEvent() for _ in range(reps)]
    for i in range(reps):
        if between is not None:
            between()
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return float(np.median([s.elapsed_time(e) for s, e in zip(starts, ends)]))


class HipEvent:
    """A HIP timing event without the system-scope fence of torch's events
    (hipEventCreateWithFlags(hipEventDisableSystemFence)): reaching it does
    not write back and invalidate the caches, which leaves less idle time
    before the next kernel."""
    _hip = None

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch loaded
        self._c = ctypes
        self.h = ctypes.c_void_p()
        rc = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h), ctypes.c_uint(0x20000000))
        assert rc == 0, f"hipEventCreateWithFlags: {rc}"

    def record(self, stream):
        rc = HipEvent._hip.hipEventRecord(self.h, self._c.c_void_p(stream.cuda_stream))
        assert rc == 0, f"hipEventRecord: {rc}"

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (waits for `end`)."""
        rc = HipEvent._hip.hipEventSynchronize(end.h)
        assert rc == 0, f"hipEventSynchronize: {rc}"
        t = self._c.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(self._c.byref(t), self.h, end.h)
        assert rc == 0, f"hipEventElapsedTime: {rc}"
        return t.value

    def __del__(self):
        if HipEvent._hip is not None and self.h:
            HipEvent._hip.hipEventDestroy(self.h)


def kernel_times(fn, reps):
    """Per-launch GPU times (ms) of the attention kernel of `reps` forward
    calls fn(), from the event pair that the library attaches to that
    kernel's dispatch (the attn_profile session of the C ABI): the RoPE table
    build and key rotation of a call are outside them."""
    xa.attn_profile_begin()
    for _ in range(reps):
        fn()
    t = xa.attn_profile_end(cap=reps)
    assert len(t) == reps, (len(t), reps)
    return t


def settle(fn, seconds):
    """Run fn back to back, untimed, for about `seconds`; returns the call count.

    Under a sustained load the GPU moves its clocks over tens to hundreds of
    milliseconds (up at first, down when a heavier kernel starts), so each
    measurement is preceded by its own workload run long enough that the
    timed calls see the clocks that workload holds when it runs continuously."""
    t_end = time.perf_counter() + seconds
    n = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        n += 8
    return n


def host_cpu():
    """The host CPU's model name (from /proc/cpuinfo), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(prefill, dec_inputs, budget_s):
    """The fp64 oracle as it stands, timed on this host on a bounded sample:
    prefill (batch, head) units in rounds of one per thread until two thirds of
    the budget are spent (or the workload is done), then whole passes of the
    decode workload for the last third (at least one pass)."""
    import oracle
    # the GPU host gives one GPU's job a share of 16 cores, whatever the
    # affinity mask shows; both numbers are reported
    avail = len(os.sched_getaffinity(0))
    threads = max(1, min(16, avail))
    cfg = W.C4
    q, k, v = prefill
    n_units = cfg.B * cfg.Hq
    done = 0
    t0 = time.perf_counter()
    while done < n_units and (done == 0 or time.perf_counter() - t0 < budget_s * 2 / 3):
        # one (batch, head) per thread: the whole 4096 x 4096 score matrix each
        units = list(range(done, min(done + threads, n_units)))
        oracle.attn_fwd(q, k, v, causal=True, scale=cfg.scale, rope_base=cfg.rope_base,
                        units=units, nthreads=threads)
        done += len(units)
    t_pre = time.perf_counter() - t0
    flops = cfg.flops / n_units * done
    out = {"value": flops / t_pre / 1e12, "unit": "TFLOP/s", "cores": threads,
           "cores_in_affinity_mask": avail, "kind": "oracle",
           "sample": f"LFM2 GQA prefill, {done} of {n_units} (batch, head) units "
                     f"(all 4096 query rows each), {t_pre:.1f} s",
           "host": host_cpu()}
    qd, kc, vc, sl = dec_inputs
    dcfg = W.C5
    all_units = list(range(dcfg.B * dcfg.Hq))
    # each unit reads its kv head's L_b rows of K and V once
    pass_bytes = sum(int(sl[u // dcfg.Hq]) * dcfg.D * 2 * 2 for u in all_units)
    passes = 0
    t0 = time.perf_counter()
    while passes == 0 or time.perf_counter() - t0 < budget_s / 3:
        oracle.decode(qd, kc, vc, sl, scale=dcfg.scale, units=all_units, nthreads=threads)
        passes += 1
    t_dec = time.perf_counter() - t0
    out["decode"] = {"value": pass_bytes * passes / t_dec / 1e9, "unit": "GB/s",
                     "sample": f"split-KV decode, {passes} pass(es) over all "
                               f"{len(all_units)} (batch, head) units, {t_dec:.1f} s"}
    return out


COPY_BYTES = 256 << 20  # calibration copy: reads and writes this many bytes
FLUSH_BYTES = 512 << 20  # written between decode repetitions (twice the 256 MiB MALL)


def profile_kernel(reps, workload, settle_s=0.5):
    """For trace and counter runs: production attn_fwd calls on the named
    prefill workload (default the LFM2 prefill: RoPE table once, then per
    call the key rotation and the fused attention kernel), back to back for
    `settle_s` seconds so the clocks settle and then `reps` more (every call
    is the same production call), then `reps` launches of a plain
    elementwise copy of COPY_BYTES (dst = src + 0) for calibration."""
    pc = {c.name: c for c in W.PREFILL}[workload]
    q_np, k_np, v_np = W.prefill_inputs(pc)
    q, k, v = W.to_device(q_np), W.to_device(k_np), W.to_device(v_np)
    o = torch.empty_like(q)
    lse = torch.empty((pc.B, pc.Hq, pc.Sq), dtype=torch.float32, device="cuda")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    def call():
        xa.attn_fwd(q, k, v, causal=pc.causal, scale=pc.scale, rope_base=pc.rope_base, o=o,
                    lse=lse)
    n_settle = settle(call, settle_s)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    log(f"profile-kernel: {n_settle} settle calls, then {reps} calls")
    for _ in range(reps):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    log("profile-kernel done")


def profile_decode(reps, ns=16):
    """For trace and counter runs: split-KV decode calls (split + merge, `ns`
    splits) on the decode workload, back to back for 0.3 s and then `reps`
    more (all at `ns` splits), then `reps` launches of the calibration
    copy."""
    dc = W.C5
    dq_np, kc_np, vc_np, sl_np = W.decode_inputs(dc)
    dq, kc, vc = W.to_device(dq_np), W.to_device(kc_np), W.to_device(vc_np)
    sl = torch.from_numpy(sl_np).cuda()
    do = torch.empty_like(dq)
    ws = torch.empty(xa.attn_decode_workspace_bytes(dc.B, dc.Hq, dc.D, ns), dtype=torch.uint8,
                     device="cuda")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    def call():
        xa.attn_decode_splitkv(dq, kc, vc, sl, ns, scale=dc.scale, o=do, workspace=ws)
    n_settle = settle(call, 0.3)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    log(f"profile-decode: {n_settle} settle calls, then {reps} calls at {ns} splits")
    for _ in range(reps):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    kv_bytes = int(sl_np.astype(np.int64).sum()) * dc.Hkv * dc.D * 2 * 2
    log(f"profile-decode done (algorithmic KV bytes per call {kv_bytes})")


def profile_backward(reps):
    """For counter runs: `reps` calls of attn_bwd on the LFM2 prefill workload
    (causal, RoPE), after the forward that gives its O and LSE."""
    pc = W.C4
    q_np, k_np, v_np = W.prefill_inputs(pc)
    q, k, v = W.to_device(q_np), W.to_device(k_np), W.to_device(v_np)
    dout = W.to_device(W.f32_to_bf16_bits(
        np.random.default_rng(pc.seed + 7).standard_normal(q_np.shape, dtype=np.float32)))
    o, lse = xa.attn_fwd(q, k, v, causal=True, scale=pc.scale, rope_base=pc.rope_base)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    torch.cuda.synchronize()
    for _ in range(reps):
        xa.attn_bwd(q, k, v, o, dout, lse, causal=True, scale=pc.scale, rope_base=pc.rope_base,
                    dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    log("profile-backward done")


def counters_summary(csv_path, match, out_path, title, cmds):
    """Per-dispatch means of every counter in a rocprofv3 counter_collection
    CSV for the kernels whose name contains `match`, with the calibration
    copy's FETCH_SIZE / WRITE_SIZE when present."""
    import csv
    vals, copy = {}, {}
    for path in csv_path.split(","):
        for r in csv.DictReader(open(path)):
            name, cn = r["Kernel_Name"], r["Counter_Name"]
            if match in name:
                vals.setdefault(cn, []).append(float(r["Counter_Value"]))
            elif "elementwise" in name and "add" in name.lower():  # the copy, not the fill
                copy.setdefault(cn, []).append(float(r["Counter_Value"]))
    lines = [f"# {title}", "# Per-dispatch means over the matching dispatches "
             f"(kernel name containing '{match}').", "# Commands (from the repository root, "
             "TMPDIR=/tmp):", *[f"#   {c}" for c in cmds]]
    if match.startswith(KERNEL_NAME):
        lines.append(f"kernel_source_sha256_16: {kernel_hash()}")
    for cn in sorted(vals):
        lines.append(f"{cn}: {np.mean(vals[cn]):.6g}  (dispatches: {len(vals[cn])})")
    for cn in sorted(copy):
        lines.append(f"calibration_copy_{cn}: {np.mean(copy[cn]):.6g}  "
                     f"(copy of {COPY_BYTES} bytes)")
    # byte counters (KiB per dispatch) scaled by expected / measured for the copy
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        if cn in vals and copy.get(cn) and np.mean(copy[cn]) > 0:
            fac = COPY_BYTES / 1024 / np.mean(copy[cn])
            lines.append(f"{cn}_bytes_per_dispatch_scaled: {np.mean(vals[cn]) * fac * 1024:.0f}"
                         f"  (scale {fac:.4f})")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_summary(csv_path, out_path, title, cmds):
    """Writes a per-kernel table (calls, average / min / max duration in us,
    share of the total) from a rocprofv3 --stats kernel_stats.csv."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))

    def col(r, *names):
        for n in names:
            if n in r:
                return r[n]
        raise KeyError(names)
    table = []
    for r in rows:
        table.append((col(r, "Name", "KernelName", "Kernel_Name"), int(float(col(r, "Calls"))),
                      float(col(r, "AverageNs")) / 1e3, float(col(r, "MinNs")) / 1e3,
                      float(col(r, "MaxNs")) / 1e3, float(col(r, "Percentage"))))
    table.sort(key=lambda t: -t[1] * t[2])
    try:  # readable names (the trace keeps some mangled); argument lists dropped
        import subprocess
        # this c++filt does not know the __bf16 / _Float16 manglings: spell
        # them as vendor types it prints by name
        raw = [t[0].replace("DF16b", "u6__bf16").replace("DF16_", "u8_Float16") for t in table]
        dem = subprocess.run(["c++filt"], input="\n".join(raw), text=True,
                             capture_output=True, check=True).stdout.splitlines()
        dem = [d[5:] if d.startswith("void ") else d for d in dem]
        table = [(d.split("(")[0] if "<" in d else d,) + t[1:] for d, t in zip(dem, table)]
    except (OSError, subprocess.CalledProcessError):
        pass
    lines = [f"# {title}", "# Commands (from the repository root, TMPDIR=/tmp):",
             *[f"#   {c}" for c in cmds], "# Durations are per dispatch, in microseconds.", "",
             f"{'kernel':90s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} "
             f"{'share%':>7s}"]
    for name, calls, avg, mn, mx, share in table:
        short = name if len(name) <= 90 else name[:87] + "..."
        lines.append(f"{short:90s} {calls:6d} {avg:9.2f} {mn:9.2f} {mx:9.2f} {share:7.2f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_summary(fetch_csv, write_csv, out_path, cmds):
    """Writes the traffic summary read by read_traffic() from two rocprofv3
    counter_collection CSVs (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch).
    Each counter is scaled by expected / measured for the calibration copy."""
    import csv

    def per_dispatch(path, counter):
        vals = {"attn": [], "copy": []}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            is_copy = "elementwise" in name and "add" in name.lower()  # not the fill of src
            key = "attn" if KERNEL_NAME in name else ("copy" if is_copy else None)
            if key:
                vals[key].append(float(r["Counter_Value"]))
        return {k_: float(np.mean(v_)) for k_, v_ in vals.items() if v_}

    fe, wr = per_dispatch(fetch_csv, "FETCH_SIZE"), per_dispatch(write_csv, "WRITE_SIZE")
    exp_kib = COPY_BYTES / 1024
    f_fac, w_fac = exp_kib / fe["copy"], exp_kib / wr["copy"]
    fetch_b, write_b = fe["attn"] * f_fac * 1024, wr["attn"] * w_fac * 1024
    pc = W.C4
    lines = [
        f"# HBM traffic of the prefill kernel {KERNEL_LABEL} on the LFM2",
        "# prefill workload (B4 Hq32 Hkv8 S4096 D64 bf16, causal, RoPE; production calls), per launch.",
        "# Counters are KiB per dispatch; each is scaled by expected/measured for a plain",
        f"# elementwise copy of {COPY_BYTES} bytes (read {COPY_BYTES}, write {COPY_BYTES}).",
        "# Commands (from the repository root, TMPDIR=/tmp):",
        *[f"#   {c}" for c in cmds],
        f"kernel_source_sha256_16: {kernel_hash()}",
        f"fetch_kib_per_launch_raw: {fe['attn']:.1f}",
        f"write_kib_per_launch_raw: {wr['attn']:.1f}",
        f"copy_fetch_kib_raw: {fe['copy']:.1f}",
        f"copy_write_kib_raw: {wr['copy']:.1f}",
        f"fetch_scale: {f_fac:.4f}",
        f"write_scale: {w_fac:.4f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"algorithmic_bytes_per_launch: {pc.io_bytes}",
        f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
    ]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle", type=float, default=0.5, metavar="SECONDS",
                    help="untimed steps for this long before the warmup steps (clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=24.0)
    ap.add_argument("--profile-workload", default=W.C4.name,
                    choices=[c.name for c in W.PREFILL],
                    help="prefill workload of --profile-kernel")
    ap.add_argument("--profile-kernel", type=int, default=0, metavar="REPS",
                    help="only launch the prefill kernel REPS times, then a calibration copy")
    ap.add_argument("--profile-settle", type=float, default=0.5, metavar="SECONDS",
                    help="untimed production calls before --profile-kernel's REPS")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 counter CSVs")
    ap.add_argument("--traffic-cmd", action="append", default=[],
                    help="command line recorded in the traffic summary (repeatable)")
    ap.add_argument("--profile-decode", type=int, default=0, metavar="REPS",
                    help="only run the split-KV decode REPS times, then a calibration copy")
    ap.add_argument("--profile-splits", type=int, default=16,
                    help="split count of --profile-decode")
    ap.add_argument("--profile-backward", type=int, default=0, metavar="REPS",
                    help="only run the LFM2 prefill backward REPS times")
    ap.add_argument("--counters-summary", nargs=4, metavar=("CSV", "MATCH", "OUT", "TITLE"),
                    help="write per-dispatch counter means of kernels matching MATCH")
    ap.add_argument("--stats-summary", nargs=3, metavar=("CSV", "OUT", "TITLE"),
                    help="write the per-kernel table of a rocprofv3 --stats kernel_stats.csv")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, TRAFFIC_FILE, args.traffic_cmd)
        return
    if args.counters_summary:
        counters_summary(*args.counters_summary, args.traffic_cmd)
        return
    if args.stats_summary:
        stats_summary(*args.stats_summary, args.traffic_cmd)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.profile_kernel:
        profile_kernel(args.profile_kernel, args.profile_workload, args.profile_settle)
        return
    if args.profile_decode:
        profile_decode(args.profile_decode, args.profile_splits)
        return
    if args.profile_backward:
        profile_backward(args.profile_backward)
        return
    stream = torch.cuda.current_stream()

    # ---- inputs, resident in HBM before anything is timed
    pc, dc = W.C4, W.C5
    log("generating inputs")
    q_np, k_np, v_np = W.prefill_inputs(pc)
    q, k, v = W.to_device(q_np), W.to_device(k_np), W.to_device(v_np)
    o = torch.empty_like(q)
    lse = torch.empty((pc.B, pc.Hq, pc.Sq), dtype=torch.float32, device="cuda")
    dq_np, kc_np, vc_np, sl_np = W.decode_inputs(dc)
    dq, kc, vc = W.to_device(dq_np), W.to_device(kc_np), W.to_device(vc_np)
    sl = torch.from_numpy(sl_np).cuda()
    do = torch.empty_like(dq)
    dlse = torch.empty((dc.B, dc.Hq), dtype=torch.float32, device="cuda")
    kv_bytes = int(sl_np.astype(np.int64).sum()) * dc.Hkv * dc.D * 2 * 2
    ws = {ns: torch.empty(xa.attn_decode_workspace_bytes(dc.B, dc.Hq, dc.D, ns),
                          dtype=torch.uint8, device="cuda") for ns in dc.splits}

    def prefill():
        xa.attn_fwd(q, k, v, causal=True, scale=pc.scale, rope_base=pc.rope_base, o=o, lse=lse)

    def decode(ns):
        xa.attn_decode_splitkv(dq, kc, vc, sl, ns, scale=dc.scale, o=do, lse=dlse,
                               workspace=ws[ns])

    # ---- settle (a fresh process's first 10-call block of the prefill runs
    # ~25 % slower than its steady state): untimed steps for `--settle` seconds
    log("settle")
    n_settle = settle(lambda: (prefill(), decode(dc.splits[0])), args.settle)

    # ---- warmup, and the split count for the decode half (outside the timed
    # region): each count timed as the decode record below is, median of
    # calls with a 512 MiB read flush before each: a reduction over a
    # 512 MiB buffer (twice the MALL) evicts the caches without leaving
    # dirty lines behind (a write flush would leave the MALL full of them,
    # and their write-back would then compete with the decode's reads)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda")

    def flush_caches():
        torch.sum(flush, dim=0, out=flush_sink)

    log("warmup")
    for _ in range(max(args.warmup, 1)):
        prefill()
        for ns in dc.splits:
            decode(ns)
    torch.cuda.synchronize()
    split_ms = {ns: timed(lambda: decode(ns), 15, stream, flush_caches) for ns in dc.splits}
    best_ns = min(split_ms, key=split_ms.get)
    log("decode ms per split count:", {k_: round(v_, 4) for k_, v_ in split_ms.items()})

    # ---- timed region: exactly `steps` steps' work, as `steps` prefill calls
    # back to back, then `steps` decode calls, events at the three boundaries
    ev = [HipEvent() for _ in range(3)]
    settle(prefill, args.settle / 5)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        prefill()
    ev[1].record(stream)
    for i in range(args.steps):
        decode(best_ns)
    ev[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = ev[0].elapsed_time(ev[1]) / args.steps
    step_dec_ms = ev[1].elapsed_time(ev[2]) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    pre_tflops = pc.flops / (pre_ms * 1e-3) / 1e12

    # ---- decode as the measurement protocol times it: 50 calls at the chosen
    # split count, each after a 512 MiB read flush (outside its events), median
    settle(lambda: decode(best_ns), args.settle / 5)
    dec_ms = timed(lambda: decode(best_ns), 50, stream, flush_caches)
    dec_gbps = kv_bytes / (dec_ms * 1e-3) / 1e9

    # ---- the dominant kernel: the fused RoPE attention kernel of the headline
    # call, timed by the library's event pair around its launch (the cached
    # RoPE table and the key-rotation pass of each call are outside the pair),
    # over max(steps, 50) production calls; median.
    settle(prefill, args.settle / 5)
    kern_all = kernel_times(prefill, max(args.steps, 50))
    kern_ms = float(np.median(kern_all))
    kern_tflops = pc.flops / (kern_ms * 1e-3) / 1e12
    traffic = read_traffic(pc.io_bytes)
    # the same kernel without RoPE on pre-rotated Q and K, for context
    qr, kr = q.clone(), k.clone()
    xa.rope_apply(qr, 0, pc.rope_base)
    xa.rope_apply(kr, 0, pc.rope_base)
    torch.cuda.synchronize()
    nr_ms = float(np.median(kernel_times(
        lambda: xa.attn_fwd(qr, kr, v, causal=True, scale=pc.scale, o=o, lse=lse),
        max(args.steps, 50))))
    del qr, kr

    # ---- backward of the same prefill (next to the hot path, not in `value`):
    # attn_bwd with the forward's O and LSE and a resident upstream gradient.
    # Algorithmic flops = 2.5 x the forward's (the recomputed S, dP, dV, dK, dQ
    # products against the forward's S and O); the kernels recompute S and dP
    # once more for dQ, which is not counted.
    dout = W.to_device(W.f32_to_bf16_bits(
        np.random.default_rng(pc.seed + 7).standard_normal(q_np.shape, dtype=np.float32)))
    xa.attn_fwd(q, k, v, causal=True, scale=pc.scale, rope_base=pc.rope_base, o=o, lse=lse)
    bwd_ws = torch.empty(xa.attn_bwd_workspace_bytes(pc.B, pc.Hq, pc.Hkv, pc.Sq, pc.Skv, pc.D,
                                                     pc.rope_base), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def backward():
        xa.attn_bwd(q, k, v, o, dout, lse, causal=True, scale=pc.scale, rope_base=pc.rope_base,
                    dq=dq, dk=dk, dv=dv, workspace=bwd_ws)
    settle(backward, args.settle / 2)
    bwd_ms = timed(backward, max(args.steps // 2, 10), stream)
    bwd_tflops = 2.5 * pc.flops / (bwd_ms * 1e-3) / 1e12

    # ---- the same prefill as four 1024-token chunks through a KV cache
    # (attn_prefill_kvcache: append + attention per chunk); same flops as the
    # one-shot prefill.
    CH = 1024
    kc_, vc_ = torch.empty_like(k), torch.empty_like(v)
    lens = torch.zeros(pc.B, dtype=torch.int32, device="cuda")
    qch = [q[:, c0:c0 + CH].contiguous() for c0 in range(0, pc.Sq, CH)]
    kch = [k[:, c0:c0 + CH].contiguous() for c0 in range(0, pc.Sq, CH)]
    vch = [v[:, c0:c0 + CH].contiguous() for c0 in range(0, pc.Sq, CH)]
    och = [torch.empty_like(x) for x in qch]

    def chunked():
        lens.zero_()
        for i in range(len(qch)):
            xa.attn_prefill_kvcache(qch[i], kch[i], vch[i], kc_, vc_, lens, causal=True,
                                    scale=pc.scale, rope_base=pc.rope_base, o=och[i],
                                    want_lse=False)
            lens.add_(CH)
    settle(chunked, args.settle / 2)
    ch_ms = timed(chunked, max(args.steps // 2, 10), stream)
    ch_tflops = pc.flops / (ch_ms * 1e-3) / 1e12

    # ---- the same prefill with a shared additive fp32 mask [S, S] (attn_fwd_masked,
    # broadcast over batch and heads by zero strides): a distance bias with a
    # 2048-key window, on top of the causal flag; same flops as the prefill.
    ii = torch.arange(pc.Sq, device="cuda", dtype=torch.float32)
    dist = ii[:, None] - ii[None, :]
    bias = torch.where(dist < 2048, -dist / 512.0, torch.full_like(dist, -float("inf")))
    del ii, dist

    def masked():
        xa.attn_fwd_masked(q, k, v, bias, causal=True, scale=pc.scale, rope_base=pc.rope_base,
                           o=o, lse=lse)
    settle(masked, args.settle / 2)
    mk_ms = timed(masked, max(args.steps // 2, 10), stream)
    mk_tflops = pc.flops / (mk_ms * 1e-3) / 1e12

    # ---- the other prefill workloads (the parity cases' shapes): the
    # attention kernel's GPU time per call (library event pairs, median of
    # max(steps, 50)), for a single fp32 head (fp32 VALU path), MHA at 1024
    # tokens without and with the causal mask, the Whisper-encoder shape
    others = {}
    for c in (W.C1, W.C2N, W.C2C, W.C3):
        qo_, ko_, vo_ = (W.to_device(x) for x in W.prefill_inputs(c))
        oo_ = torch.empty_like(qo_)
        lo_ = torch.empty((c.B, c.Hq, c.Sq), dtype=torch.float32, device="cuda")

        def call(c=c, qo_=qo_, ko_=ko_, vo_=vo_, oo_=oo_, lo_=lo_):
            xa.attn_fwd(qo_, ko_, vo_, causal=c.causal, scale=c.scale, o=oo_, lse=lo_)
        settle(call, args.settle / 5)
        c_ms = float(np.median(kernel_times(call, max(args.steps, 50))))
        c_tf = c.flops / (c_ms * 1e-3) / 1e12
        others[c.name] = {"shape": f"B{c.B} Hq{c.Hq} Hkv{c.Hkv} S{c.Sq} D{c.D} {c.dtype}"
                                   f"{' causal' if c.causal else ''}",
                          "ms": round(c_ms, 4), "tflops": round(c_tf, 3),
                          "frac_of_peak": round(c_tf / (PEAK_F32_TFLOPS if c.dtype == "f32"
                                                        else PEAK_BF16_TFLOPS), 4)}
        del qo_, ko_, vo_, oo_, lo_

    result = {
        "metric": METRIC,
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "LFM2-2.6B-shaped GQA prefill B4 Hq32 Hkv8 S4096 D64 causal RoPE-10000 "
                        "+ split-KV decode B16 Hq32 Hkv8 D128 Smax32768 L~U[1024,32768]",
            "prefill": {"B": pc.B, "Hq": pc.Hq, "Hkv": pc.Hkv, "S": pc.Sq, "D": pc.D,
                        "causal": True, "rope_base": pc.rope_base, "seed": pc.seed},
            "decode": {"B": dc.B, "Hq": dc.Hq, "Hkv": dc.Hkv, "D": dc.D, "Smax": dc.Smax,
                       "sum_lengths": int(sl_np.sum()), "num_splits": best_ns, "seed": dc.seed},
            "parallelism": "single GPU",
            "settle": {"seconds": args.settle, "untimed_steps": n_settle,
                       "seconds_before_backward_chunked_masked": args.settle / 2},
        },
        "prefill": {"what": "whole attn_fwd call (key rotation + attention kernel; RoPE table "
                            "cached): the timed region's prefill run of `steps` calls between "
                            "two events, per call",
                    "ms": round(pre_ms, 4),
                    "tflops": round(pre_tflops, 2),
                    "frac_of_mfma_peak": round(pre_tflops / PEAK_BF16_TFLOPS, 4)},
        "decode": {"what": f"attn_decode_splitkv (split + merge) at {best_ns} splits, 50 calls "
                           f"each after a {FLUSH_BYTES >> 20} MiB read flush outside the "
                           "events, median",
                   "ms": round(dec_ms, 4), "GBps": round(dec_gbps, 1),
                   "frac_of_hbm_peak": round(dec_gbps / PEAK_HBM_GBPS, 4),
                   "kv_bytes": kv_bytes,
                   "ms_in_timed_region": round(step_dec_ms, 4),
                   "ms_in_timed_region_what": "the timed region's decode run of `steps` calls "
                                              "back to back (no flush) between two events, "
                                              "per call",
                   "ms_by_splits": {str(k_): round(v_, 4) for k_, v_ in split_ms.items()}},
        "roofline": {"kernel": KERNEL_LABEL, "bound": "mfma",
                     "achieved": round(kern_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
                     "launch_ms": round(kern_ms, 4),
                     "launch_ms_mean": round(float(np.mean(kern_all)), 4),
                     "timing": "HIP event pair attached by the library to the kernel's dispatch "
                               "(hipExtLaunchKernel; attn_profile session), median",
                     "traffic": traffic,
                     "no_rope_variant": {"kernel": KERNEL_LABEL_NOROPE,
                                         "launch_ms": round(nr_ms, 4),
                                         "frac": round(pc.flops / (nr_ms * 1e-3) / 1e12 /
                                                       PEAK_BF16_TFLOPS, 4)}},
        "backward": {"workload": "LFM2 GQA prefill backward (dq, dk, dv), RoPE, causal",
                     "ms": round(bwd_ms, 4), "tflops": round(bwd_tflops, 2),
                     "frac_of_mfma_peak": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "flops": "2.5 x forward (5 products)"},
        "chunked_prefill": {"workload": "LFM2 GQA prefill as 4 chunks of 1024 tokens through "
                                        "a KV cache (append + attention per chunk)",
                            "ms": round(ch_ms, 4), "tflops": round(ch_tflops, 2),
                            "frac_of_mfma_peak": round(ch_tflops / PEAK_BF16_TFLOPS, 4)},
        "masked_prefill": {"workload": "LFM2 GQA prefill with a shared [4096, 4096] fp32 "
                                       "additive mask (distance bias, 2048-key window), causal",
                           "ms": round(mk_ms, 4), "tflops": round(mk_tflops, 2),
                           "frac_of_mfma_peak": round(mk_tflops / PEAK_BF16_TFLOPS, 4)},
        "other_prefill_workloads": others,
        "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbps, 1),
                            "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                            "frac": round(dec_gbps / PEAK_HBM_GBPS, 4)},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        result["cpu_baseline"] = cpu_baseline((q_np, k_np, v_np), (dq_np, kc_np, vc_np, sl_np),
                                              args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
