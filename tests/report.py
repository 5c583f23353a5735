"""Per-workload results records: one JSON file per workload with its parity
against the fp64 oracle, its GPU timing, throughput and roofline fraction,
the oracle's own time and thread count, and the rocprofv3 summaries behind
the numbers.

This is test infrastructure (it runs the oracle), used as a script on a
machine with the GPU:

    python3 bench.py > gpurun_out/bench.log
    python3 tests/report.py --bench gpurun_out/bench.log --out gpurun_out/results

For every workload (single fp32 head, 1024-token MHA non-causal and causal,
Whisper encoder, LFM2 GQA prefill, split-KV decode) it runs the library once
on the seeded inputs, runs the oracle on every (batch, head) unit of the same
inputs (timed), and compares every element of O and LSE: O max-abs error,
O relative L2 error, LSE max-abs error, against the bars the parity tests
enforce (fp32 1e-4 / 1e-4; 16-bit 2e-2 max-abs and 5e-3 rel-L2 on O, 1e-3 on
the LSE).  Timings, throughput and roofline fractions are copied from the
benchmark's JSON line (the library's own event timings, taken on the same
machine); the counter figures are read from the committed summaries under
profiles/ that cover the workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import exact_attention_28_amd as xa  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

# the committed rocprofv3 summaries that cover each workload
PROFILES = {
    "single_head_f32": [],
    "mha_s1024": ["fwdp_mha_s1024_kernel_stats.txt", "fwdp_mha_s1024_sq_counters.txt"],
    "mha_s1024_causal": ["fwdp_mha_s1024_causal_kernel_stats.txt"],
    "whisper_encoder_s1500": ["fwdp_whisper_encoder_s1500_kernel_stats.txt",
                              "fwdp_whisper_encoder_s1500_sq_counters.txt"],
    "lfm2_gqa_prefill_s4096": ["fwdp_lfm2_gqa_prefill_s4096_kernel_stats.txt",
                               "fwdp_lfm2_gqa_prefill_s4096_sq_counters.txt",
                               "fwdp_lfm2_gqa_prefill_s4096_traffic.txt"],
    "splitkv_decode_s32768": ["decode_splitkv_s32768_ns16_kernel_stats.txt",
                              "decode_split_splitkv_s32768_traffic.txt"],
}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def parity(o, lse, o_ref, lse_ref, fp32):
    """Element-by-element comparison of every O and LSE value."""
    o = np.asarray(o, np.float64)
    err = np.abs(o - o_ref)
    rel = float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-30))
    fin = np.isfinite(lse_ref)
    same_fin = bool((np.isfinite(lse) == fin).all())
    lerr = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    bar = ({"o_max_abs": 1e-4, "lse_max_abs": 1e-4} if fp32 else
           {"o_max_abs": 2e-2, "o_rel_l2": 5e-3, "lse_max_abs": 1e-3})
    ok = (bool(np.isfinite(o).all()) and same_fin and err.max() <= bar["o_max_abs"]
          and lerr <= bar["lse_max_abs"] and rel <= bar.get("o_rel_l2", np.inf))
    return {"o_elements": int(o.size), "lse_elements": int(lse_ref.size),
            "o_max_abs": float(err.max()), "o_rel_l2": rel, "lse_max_abs": lerr,
            "lse_finite_pattern_equal": same_fin, "bar": bar, "pass": bool(ok)}


def read_profiles(name):
    """The figures of each committed summary: 'key: value' lines and the rows
    of kernel-stat tables (kernel name -> calls, avg/min/max us, share)."""
    out = {}
    for fn in PROFILES[name]:
        path = os.path.join(ROOT, "profiles", fn)
        if not os.path.exists(path):
            continue
        figs, kernels = {}, {}
        table = fn.endswith("kernel_stats.txt")
        with open(path) as f:
            for ln in f:
                ln = ln.rstrip("\n")
                if not ln or ln.startswith("#") or ln.startswith("kernel "):
                    continue
                if table:
                    parts = ln.split()
                    kernels[" ".join(parts[:-5])] = {
                        "calls": int(parts[-5]), "avg_us": float(parts[-4]),
                        "min_us": float(parts[-3]), "max_us": float(parts[-2]),
                        "share_pct": float(parts[-1])}
                elif ":" in ln:
                    key, val = ln.split(":", 1)
                    figs[key.strip()] = val.strip()
        out[fn] = {"kernels": kernels} if table else {"figures": figs}
    return out


def bench_line(path):
    with open(path) as f:
        for ln in f:
            ln = ln.strip()
            if ln.startswith("{") and '"metric"' in ln:
                return json.loads(ln)
    raise SystemExit(f"no benchmark JSON line in {path}")


def gpu_figures(name, bench):
    """The benchmark's timing of this workload."""
    if name == "lfm2_gqa_prefill_s4096":
        rf = bench["roofline"]
        return {"call": bench["prefill"], "kernel": {k: rf[k] for k in (
            "kernel", "launch_ms", "achieved", "unit", "frac", "traffic") if k in rf}}
    if name == "splitkv_decode_s32768":
        return {"call": bench["decode"], "roofline": bench["roofline_decode"]}
    return {"call": bench["other_prefill_workloads"][name]}


def prefill_record(cfg, bench):
    q, k, v = W.prefill_inputs(cfg)
    o, lse = xa.attn_fwd(W.to_device(q), W.to_device(k), W.to_device(v), causal=cfg.causal,
                         scale=cfg.scale, rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale,
                                     rope_base=cfg.rope_base, nthreads=THREADS)
    t_or = time.perf_counter() - t0
    # the oracle forms every full score matrix: 4 B Hq Sq Skv D flops, causal or not
    or_flops = 4 * cfg.B * cfg.Hq * cfg.Sq * cfg.Skv * cfg.D
    return {
        "workload": cfg.name,
        "shape": {"B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "Sq": cfg.Sq, "Skv": cfg.Skv,
                  "D": cfg.D, "causal": cfg.causal, "rope_base": cfg.rope_base,
                  "dtype": cfg.dtype, "seed": cfg.seed, "input_amplitude": cfg.amplitude},
        "algorithmic_flops": cfg.flops,
        "parity": parity(_np(o), _np(lse), o_ref, lse_ref, cfg.dtype == "f32"),
        "gpu": gpu_figures(cfg.name, bench),
        "oracle": {"seconds": t_or, "threads": THREADS, "fp64_gflops": or_flops / t_or / 1e9,
                   "what": "every (batch, head) unit, full score matrices in fp64"},
        "profiles": read_profiles(cfg.name),
    }


def decode_record(cfg, bench):
    q, kc, vc, sl = W.decode_inputs(cfg)
    dev = (W.to_device(q), W.to_device(kc), W.to_device(vc), torch.from_numpy(sl).cuda())
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.decode(q, kc, vc, sl, scale=cfg.scale, nthreads=THREADS)
    t_or = time.perf_counter() - t0
    par = {}
    for ns in cfg.splits:
        o, lse = xa.attn_decode_splitkv(*dev, ns, scale=cfg.scale)
        torch.cuda.synchronize()
        par[str(ns)] = parity(_np(o), _np(lse), o_ref, lse_ref, False)
    kv_bytes = int(sl.astype(np.int64).sum()) * cfg.Hkv * cfg.D * 2 * 2
    return {
        "workload": cfg.name,
        "shape": {"B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D, "Smax": cfg.Smax,
                  "lengths": [cfg.len_lo, cfg.len_hi], "sum_lengths": int(sl.sum()),
                  "seed": cfg.seed, "dtype": "bf16"},
        "algorithmic_kv_bytes": kv_bytes,
        "parity_by_splits": par,
        "gpu": gpu_figures(cfg.name, bench),
        "oracle": {"seconds": t_or, "threads": THREADS, "GBps": kv_bytes / t_or / 1e9,
                   "what": "every (batch, query head) unit"},
        "profiles": read_profiles(cfg.name),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--bench", required=True, help="file holding bench.py's JSON line")
    ap.add_argument("--out", required=True, help="directory for <workload>.json")
    a = ap.parse_args()
    bench = bench_line(a.bench)
    os.makedirs(a.out, exist_ok=True)
    host = {"cpu_threads_used": THREADS, "cpu_threads_in_affinity_mask":
            len(os.sched_getaffinity(0)), "gpu": torch.cuda.get_device_name(0)}
    cmd = "python3 tests/report.py --bench <bench.py output> --out <dir>"
    for cfg in list(W.PREFILL) + [W.C5]:
        print("report", cfg.name, flush=True)
        rec = prefill_record(cfg, bench) if cfg is not W.C5 else decode_record(cfg, bench)
        rec["host"] = host
        rec["command"] = cmd
        rec["bench_metric"] = bench["metric"]
        with open(os.path.join(a.out, cfg.name + ".json"), "w") as f:
            json.dump(rec, f, indent=1, sort_keys=False)
            f.write("\n")
        par = rec.get("parity") or rec["parity_by_splits"]["16"]
        print(f"  parity pass={par['pass']} O max-abs {par['o_max_abs']:.3e} "
              f"rel-L2 {par['o_rel_l2']:.3e} LSE {par['lse_max_abs']:.3e}; "
              f"oracle {rec['oracle']['seconds']:.1f} s", flush=True)


if __name__ == "__main__":
    main()
