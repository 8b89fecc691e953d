"""Prefill throughput benchmark on one MI355X.

One step = one full prefill forward (embedding, every block, final norm, lm_head) of the
StableLM-2-1.6B-shaped model (24 layers, hidden 2048, 32 heads x 64, partial RoPE 16/64,
SwiGLU 5632, vocab 100352) on a batch of 8 x 2048 synthetic token ids, fp16 weights and
activations with fp32 accumulation and fp32 logits; ids and weights are resident in HBM
before the timed region starts.

Prints ONE JSON line with tokens/s, the fraction of the fp16 dense MFMA peak reached by
the whole forward, a roofline entry for the dominant kernel (the SwiGLU gate/up GEMM,
timed with HIP events on the stream it runs on, in separate steps after the headline
ones) and the CPU oracle's throughput on a bounded sample of the same workload.

The headline region runs `--steps` forwards through the plain `tf_prefill` entry point
with nothing recorded inside a step, and is repeated once (`repeat`) in the same process.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0   # MI355X published dense fp16 MFMA peak (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM traffic of the gate/up GEMM measured with rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE runs, calibrated against a plain device copy); valid only while the GEMM
# sources are the ones it was measured on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_c2_traffic.md")
GEMM_SOURCES = [os.path.join(ROOT, "dense_transformer_prefill_amd", "csrc", f)
                for f in ("gemm_kernel.h", "k_gemm.hip")]


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """Bytes per launch from the committed counter summary, or None if it is missing or
    was taken on other GEMM sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != gemm_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class ClockSampler:
    """Samples the GPU's graphics clocks (mean over its XCDs) and socket power with
    `amd-smi metric` in a background thread; only samples taken wholly inside the timed
    region count. Reports nothing if the tool is missing or fails."""

    def __init__(self, gpu: int = 0):
        import shutil
        import threading
        self.gpu = gpu
        self.exe = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi"
                                               if os.path.exists("/opt/rocm/bin/amd-smi") else None)
        self.clk, self.pw = [], []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _sample(self):
        import subprocess
        ts = time.perf_counter()
        r = subprocess.run([self.exe, "metric", "-g", str(self.gpu), "--clock", "--power", "--json"],
                           capture_output=True, text=True, timeout=10)
        d = json.loads(r.stdout)["gpu_data"][0]
        clks = [v["clk"]["value"] for k, v in d["clock"].items()
                if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        te = time.perf_counter()
        if clks:
            self.clk.append((ts, te, sum(clks) / len(clks)))
        p = d.get("power", {}).get("socket_power", {})
        if isinstance(p, dict) and isinstance(p.get("value"), (int, float)):
            self.pw.append((ts, te, float(p["value"])))

    def _run(self):
        while not self._stop.is_set():
            try:
                self._sample()
            except Exception:
                return

    def start(self):
        if self.exe:
            self._t.start()
        return self

    def stop(self, t0: float, t1: float):
        """Summaries of the samples taken within [t0, t1] (perf_counter seconds)."""
        self._stop.set()
        if self._t.is_alive():
            self._t.join(timeout=15)
        def summ(samples, unit):
            v = [x for ts, te, x in samples if ts >= t0 and te <= t1]
            if not v:
                return None
            return {"mean": round(sum(v) / len(v), 1), "min": min(v), "max": max(v),
                    "samples": len(v), "unit": unit}
        return summ(self.clk, "MHz"), summ(self.pw, "W")


def file_sha256(path: str):
    import hashlib
    if not os.path.exists(path):
        return None
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, W, ids, sample_tokens: int, gpu_tokens_s: float):
    """Time the oracle as it stands (the plain float32 forward) on one batch row's first
    `sample_tokens` positions of the same workload -- a whole row is one GPU's
    data-parallel share -- and on its first 512 (a forward of the 1.6B shape's b1 s512
    size), with every host core this process may use."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    cores = len(os.sched_getaffinity(0))

    def run(n):
        sub = cfg.with_(batch=1, seq=n)
        with threadpool_limits(limits=cores):
            t0 = time.perf_counter()
            out = oracle.forward(sub, W, ids[:1, :n], dtype=np.float32)
            dt = time.perf_counter() - t0
        assert np.isfinite(out).all()
        return dt, sub.flops()

    dt, fl = run(sample_tokens)
    out = {"value": round(sample_tokens / dt, 3), "unit": "tokens/s", "cores": cores,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"{cfg.name}: batch row 0, positions 0..{sample_tokens - 1} "
                     f"({sample_tokens} tokens, float32 numpy oracle), {dt:.1f} s",
           "gflop_s": round(fl / dt / 1e9, 1),
           "gpu_speedup": round(gpu_tokens_s / (sample_tokens / dt), 1)}
    if sample_tokens > 512:
        dt5, fl5 = run(512)
        out["b1_s512"] = {"value": round(512 / dt5, 3), "unit": "tokens/s",
                          "seconds": round(dt5, 2), "gflop_s": round(fl5 / dt5 / 1e9, 1)}
    return out


def provenance():
    """What ran: the command line, the repository commit when a checkout is present, the
    library's own build record and whether the library was built from the sources here."""
    import subprocess
    from dense_transformer_prefill_amd import build as B
    from dense_transformer_prefill_amd import load
    head = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=10)
        head = r.stdout.strip() or None
    except Exception:
        pass
    lib_info = load().tf_build_info().decode()
    src = B.sources_sha256()
    return {"command": " ".join([os.path.basename(sys.executable)] + sys.argv),
            "git_head": head, "lib_build": lib_info, "sources_sha256": src,
            "lib_matches_sources": lib_info.startswith(f"sources {src} ")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2_stablelm2_b8s2048")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    ap.add_argument("--kernel-steps", type=int, default=5,
                    help="forwards after the headline ones in which the gate/up GEMM's "
                         "launches are timed with HIP events (roofline entry)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--padded", action="store_true",
                    help="call with an attention_mask (row r's first 200 r positions are "
                         "padding) and compute next_token_probs in every step")
    ap.add_argument("--no-clock-sampler", action="store_true",
                    help="do not sample clocks and power with amd-smi (for profiler runs, "
                         "where the preloaded profiler makes the sampler's child processes "
                         "fail)")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="before warm-up, run one plain 1 GiB device copy (the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library's path is single-GPU. Batch rows are "
              "independent sequences, so a run on N GPUs would give each GPU batch/N rows "
              "with no exchange between them; measure one GPU's share with --config.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from dense_transformer_prefill_amd import KERNEL_CLASSES, PrefillModel, upload_weights
    from workloads import CONFIGS, synth_ids, synth_weights

    cfg = CONFIGS[args.config]
    T = cfg.tokens
    W = synth_weights(cfg)
    ids_np = synth_ids(cfg)
    model = PrefillModel(cfg, upload_weights(W))
    ids = torch.from_numpy(ids_np).cuda()
    logits = torch.empty((cfg.batch, cfg.seq, cfg.vocab), dtype=torch.float32, device="cuda")
    kt = KERNEL_CLASSES["gemm_mlp_up"]
    extra = {}
    if args.padded:
        m = torch.ones((cfg.batch, cfg.seq), dtype=torch.int32)
        for r in range(cfg.batch):
            m[r, :min(200 * r, cfg.seq - 1)] = 0
        extra = dict(attention_mask=m.cuda(),
                     next_token_probs=torch.empty((cfg.batch, cfg.vocab), dtype=torch.float32,
                                                  device="cuda"))

    if args.pmc_calibrate:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        model.prefill(ids, out=logits, **extra)
    torch.cuda.synchronize()

    def timed_region(sample_clock: bool):
        """K forwards between two synchronisations; per-step torch events at the step
        boundaries only (nothing is recorded inside a forward)."""
        sampler = ClockSampler(0)
        if sample_clock and not args.no_clock_sampler:
            sampler.start()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i].record()
            model.prefill(ids, out=logits, **extra)
        ev[args.steps].record()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        clk = sampler.stop(t0, t0 + dt) if sample_clock else (None, None)
        steps = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
        return dt, steps, clk

    dt, step_ms, (sclk, power) = timed_region(True)
    dt2, step_ms2, _ = timed_region(False)
    assert torch.isfinite(logits).all().item(), "non-finite logits"

    # the dominant kernel, timed in steps of its own after the headline ones
    model.timing(kt)  # discard
    for _ in range(args.kernel_steps):
        model.prefill(ids, out=logits, timed_kernel=kt, **extra)
    torch.cuda.synchronize()

    ms_step = dt / args.steps * 1e3
    tokens_s = T * args.steps / dt
    flops = cfg.flops()
    tflops = flops / (ms_step * 1e-3) / 1e12

    k_ms, k_n = model.timing(kt)
    k_avg_ms = k_ms / max(k_n, 1)
    g = 2 if cfg.mlp_kind == "swiglu" else 1
    k_flops = 2.0 * T * cfg.hidden * g * cfg.inter   # algorithmic FLOPs per launch
    k_tflops = k_flops / (k_avg_ms * 1e-3) / 1e12

    rec = {
        "metric": ("prefill tokens/s and % of fp16 MFMA peak, StableLM-2-1.6B shape b8 s2048"
                   if cfg.name == "c2_stablelm2_b8s2048" else
                   f"prefill tokens/s and % of fp16 MFMA peak, {cfg.name}")
                  + (" (padded)" if args.padded else ""),
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 3),
        "ms_per_step_min": round(step_ms[0], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,0.02) fp16 weights, uniform token ids)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq": cfg.seq,
                   "tokens_per_step": T, "layers": cfg.n_layers, "hidden": cfg.hidden,
                   "heads": cfg.n_heads, "head_dim": cfg.head_dim, "inter": cfg.inter,
                   "vocab": cfg.vocab, "kv_heads": cfg.kv_heads,
                   "block": "parallel" if cfg.parallel_residual else
                            ("post-norm" if cfg.norm_place == "post" else "pre-norm"),
                   "qk_norm": cfg.qk_norm, "rot_dim": cfg.rot_dim, "alibi": cfg.alibi,
                   "weights": cfg.weight_format,
                   "logits": "fp32",
                   "padding": ("attention_mask, row r left-padded by 200 r; next_token_probs"
                               if args.padded else "none")},
        "repeat": {"ms_per_step": round(dt2 / args.steps * 1e3, 3),
                   "value": round(T * args.steps / dt2, 1),
                   "ms_per_step_median": round(step_ms2[len(step_ms2) // 2], 3),
                   "ms_per_step_min": round(step_ms2[0], 3)},
        "tflops": round(tflops, 1),
        "sclk_mhz": sclk, "socket_power_w": power,
        "lib_sha256": file_sha256(os.path.join(ROOT, "dense_transformer_prefill_amd",
                                               "libtf_prefill.so")),
        "frac_of_fp16_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
        "gflop_per_step": round(flops / 1e9, 1),
        "roofline": {"kernel": ("gemm gate/up + SwiGLU epilogue" if cfg.mlp_kind == "swiglu"
                                else "gemm fc1 + bias + GELU epilogue"), "bound": "mfma",
                     "achieved": round(k_tflops, 1), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(k_tflops / PEAK_FP16_TFLOPS, 4),
                     # counted on the 1.6B-shape b8 s2048 gate/up GEMM only
                     "traffic": (measured_traffic() if cfg.name == "c2_stablelm2_b8s2048"
                                 else None),
                     "launches": k_n,
                     "timed_in": f"{args.kernel_steps} forwards after the headline ones",
                     "avg_ms": round(k_avg_ms, 4),
                     "flop_per_launch": k_flops},
    }
    rec["provenance"] = provenance()
    model.close()
    del logits
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, W, ids_np, min(args.cpu_sample_tokens, cfg.seq),
                                           tokens_s)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
