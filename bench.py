"""Throughput of the GPT-2 124M training step on one MI355X.

    python bench.py [--gpus 1] [--steps 3] [--warmup 1] [--no-cpu-baseline]
    python bench.py --workload lmhead         (the isolated lm_head + loss)
    python bench.py --traffic-probe SITE     (under rocprofv3 --pmc, see below)

One step is the pages' full optimizer step: zero_grad, 32 micro-steps of
B=16 x T=1024 tokens with loss / 32, global-norm clipping at 1.0 and AdamW
(lr 6e-4, betas 0.9/0.95, eps 1e-8, wd 0.1 on 2-D tensors) -- 524,288 tokens
("How I trained my own GPT-2 124M on FineWeb-Edu" sections 8.1 and 9; the
timing protocol of "Making Training Fast on One GPU": warm-up, then timed
full steps with a device synchronisation on both sides, the loss read back
once per step).  Inputs are a synthetic Zipf token stream resident in HBM
before timing starts; weights are the library's own N(0, 0.02) init.

Prints one JSON line with tokens/s, MFU (against the bf16 peak and against
the best bf16 product this library measures on the box), the GPU clock
sampled during the timed steps, the roofline of the dominant kernel (its
launches timed with HIP events on the library's stream during the timed
steps; the per-site breakdown comes from the first warm-up step), and the
CPU oracle timed on a bounded sample on this host.  The roofline's `traffic`
(HBM bytes per launch of the dominant kernel) is read from a record under
profiles/ written by `python -m gpt_pretraining_step_amd.profiling traffic`
from two counter runs of `--traffic-probe`, and is null when no record
matches the kernel's current sources.

`--workload lmhead` times the isolated tied lm_head + cross-entropy forward
and backward (hidden [65,536 x 768], vocabulary 50,304, 10% of targets
ignored): the median of the timed calls, in TFLOP/s of its 3 x 2 M C V
algorithmic FLOPs.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15          # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12           # MI355X HBM3E, B/s

# The two measured workloads.  "gpt2" is the headline: the GPT-2 124M
# optimizer step of "How I trained my own GPT-2 124M on FineWeb-Edu" (32 x
# B=16, lr 6e-4).  "rotary" is the modern variant that "Reproduce GPT-2 124M
# 复盘" runs on one H100 (RMSNorm, RoPE, SwiGLU 2048; 8 x B=64, lr 1.5e-3).
WORKLOADS = {
    "gpt2": dict(metric="train tokens/sec + MFU %, GPT-2 124M B=16 T=1024 step, 1 MI355X", B=16, G=32, lr=6e-4,
                 F=3072, name="gpt2-124m optimizer step"),
    "rotary": dict(metric="train tokens/sec + MFU %, GPT-2 124M rotary variant B=64 T=1024 step, 1 MI355X", B=64,
                   G=8, lr=1.5e-3, F=2048, name="gpt2-124m rotary variant (RMSNorm, RoPE, SwiGLU 2048) optimizer step"),
}
T = 1024
B, G = WORKLOADS["gpt2"]["B"], WORKLOADS["gpt2"]["G"]
METRIC = WORKLOADS["gpt2"]["metric"]


def flops_per_token(n_params: int, L=12, H=12, hd=64, T_=1024) -> int:
    # "Making Training Fast on One GPU", MFU defined: 6N + 12 L H Q T
    return 6 * n_params + 12 * L * H * hd * T_


CE_CHUNK = 8192  # rows per lm_head chunk of the library (bf16)


def gemm_site_flops(rows=B * T, F=3072, FC=None, L=12):
    """Algorithmic FLOPs of one launch at each GEMM site of the micro-step
    (rows = B*T, C = 768, MLP width F, V = 50304).  FC is the fc product's
    output width: F for GPT-2, 2F (gate and up) for the rotary variant.
    gemm.dw is the grouped launch of the L blocks' four weight-gradient
    products.  The lm_head runs per chunk of CE_CHUNK rows: gemm.lm_head is
    one chunk's logits product, gemm.lm_head_bwd one chunk's dZ and dW
    products together."""
    M, C, V = rows, 768, 50304
    FC = F if FC is None else FC
    chunk = min(M, CE_CHUNK)
    return {
        "gemm.dw": L * 2 * M * C * (3 * C + C + FC + F),
        "gemm.qkv": 2 * M * 3 * C * C,
        "gemm.attn_proj": 2 * M * C * C,
        "gemm.fc": 2 * M * FC * C,
        "gemm.mlp_proj": 2 * M * C * F,
        "gemm.lm_head": 2 * chunk * V * C,
        "gemm.lm_head_bwd": 2 * 2 * chunk * V * C,
        "gemm.mlp_proj_dx": 2 * M * C * F,
        "gemm.fc_dx": 2 * M * FC * C,
        "gemm.attn_proj_dx": 2 * M * C * C,
        "gemm.qkv_dx": 2 * M * 3 * C * C,
    }


class ClockSampler:
    """The GPU's graphics clock, sampled with amd-smi from a host thread
    while the timed steps run ("Making Training Fast on One GPU", clock
    drift as noise: the clock is logged beside each timing)."""

    def __init__(self, period: float = 0.5):
        import threading
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def read_mhz():
        import subprocess
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True,
                               timeout=10)
            data = json.loads(r.stdout)
        except Exception:
            return None
        vals = []

        def walk(x, key=""):
            if isinstance(x, dict):
                for k, v in x.items():
                    if key.startswith("gfx") and k == "clk":
                        val = v.get("value") if isinstance(v, dict) else v
                        if isinstance(val, (int, float)):
                            vals.append(float(val))
                    else:
                        walk(v, k if isinstance(k, str) else "")
            elif isinstance(x, list):
                for v in x:
                    walk(v, key)
        walk(data)
        return sum(vals) / len(vals) if vals else None

    def _run(self):
        while not self._stop.is_set():
            v = self.read_mhz()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join(timeout=15)

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"gfx_mhz_median": round(v[len(v) // 2], 1), "gfx_mhz_min": round(v[0], 1),
                "gfx_mhz_max": round(v[-1], 1), "samples": len(v), "source": "amd-smi metric -c (mean over XCDs)"}


def measured_peak_tflops(reps: int = 20):
    """Measured bf16 product rates on the box, the yardstick "Making
    Training Fast on One GPU" reports MFU against beside the spec sheet's
    peak: an 8192^3 bf16 product through torch.mm (the vendor BLAS, run here
    only as a measuring stick, never in the training path) and the same
    product through this library's gpt2_op_gemm; median of `reps` launches
    each, timed with HIP events."""
    import torch
    import gpt_pretraining_step_amd as g
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    st = torch.cuda.current_stream()

    def rate(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn()
            e1.record(st)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        ts.sort()
        return 2 * n ** 3 / ts[len(ts) // 2] / 1e12

    out = {"vendor_blas_8192": round(rate(lambda: torch.mm(a, b, out=c)), 1),
           "library_8192": round(rate(lambda: g.op_gemm(a, b, c, n, n, n)), 1)}
    del a, b, c
    torch.cuda.empty_cache()
    return out


def cpu_baseline(rows: int = 8, workload: str = "gpt2"):
    """The CPU oracle (NumPy float32) on a bounded sample: one micro-step of the
    same model on `rows` 1024-token sequences of the same token stream (about
    2 s of host time per sequence on 16 cores)."""
    import synthetic
    if workload == "rotary":
        from oracle import modern as OM
        cfg = OM.ModernConfig(50304, 1024, 12, 12, 768, 2048)
        what = "the GPT-2 124M rotary variant"
    else:
        from oracle import model as OM
        cfg = OM.Config(50304, 1024, 12, 12, 768, 3072)
        what = "GPT-2 124M"
    cores = len(os.sched_getaffinity(0))
    params = synthetic.random_params(OM.param_specs(cfg), seed=42)
    stream = synthetic.token_stream(rows * 1024 + 1, seed=1337)
    x, y = synthetic.micro_batch(stream, 0, rows, 1024)
    t0 = time.perf_counter()
    OM.fwd_bwd(cfg, params, x, y, scale=1.0 / WORKLOADS[workload]["G"])
    dt = time.perf_counter() - t0
    return {"value": round(rows * 1024 / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one micro-step (forward + backward, float32 NumPy) of {what} on {rows} x 1024 tokens of "
                      f"the synthetic stream; {dt:.1f} s"}


COPY_BYTES = 256 << 20


def traffic_probe(site: str, workload: str = "gpt2") -> int:
    """One micro-step of `workload` with the library's marker kernel launched
    before every launch of `site`, then the marker and a plain device copy of
    COPY_BYTES (read and written once) that calibrates the HBM byte counters.
    Run under `rocprofv3 --pmc FETCH_SIZE` and again under `--pmc
    WRITE_SIZE`."""
    import torch
    import gpt_pretraining_step_amd as g
    import synthetic
    wl = WORKLOADS[workload]
    Bw, Gw = wl["B"], wl["G"]
    model = g.GPT2(g.GPT2_124M if workload == "gpt2" else g.GPT2_ROTARY_124M)
    model.init_params(seed=42)
    stream = synthetic.token_stream(Bw * T + 1, seed=1337)
    x, y = synthetic.micro_batch(stream, 0, Bw, T)
    x, y = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    model.zero_grad()
    torch.cuda.synchronize()
    model.profile(True)
    model.profile_only(site)
    model.profile_mark(True)
    model.fwd_bwd(x, y, loss_scale=1.0 / Gw)
    g.op_marker()
    dst.copy_(src)
    torch.cuda.synchronize()
    st = model.status()
    n = model.profile_entries().get(site, (0, 0.0))[0]
    model.close()
    print(f"[bench] traffic probe: {workload} site {site}, {n} marked launches, status {st}", file=sys.stderr,
          flush=True)
    return 0 if st == 0 and n > 0 else 1


def counter_probe(workload: str = "gpt2") -> int:
    """One micro-step of `workload` and one clip + AdamW step, then the
    library's marker kernel and a plain device copy of COPY_BYTES that
    calibrates the HBM byte counters.  Run under `rocprofv3 --pmc ...` (one
    counter set per run) and under `--kernel-trace --stats`; the summaries
    come from `python -m gpt_pretraining_step_amd.profiling counters`."""
    import torch
    import gpt_pretraining_step_amd as g
    import synthetic
    wl = WORKLOADS[workload]
    Bw, Gw = wl["B"], wl["G"]
    model = g.GPT2(g.GPT2_124M if workload == "gpt2" else g.GPT2_ROTARY_124M)
    model.init_params(seed=42)
    stream = synthetic.token_stream(Bw * T + 1, seed=1337)
    x, y = synthetic.micro_batch(stream, 0, Bw, T)
    x, y = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    model.zero_grad()
    model.fwd_bwd(x, y, loss_scale=1.0 / Gw)
    model.clip_adamw_step(lr=wl["lr"])
    g.op_marker()
    dst.copy_(src)
    torch.cuda.synchronize()
    st = model.status()
    model.close()
    print(f"[bench] counter probe: {workload} micro-step + optimizer step, status {st}", file=sys.stderr, flush=True)
    return 0 if st == 0 else 1


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--grad-accum", type=int, default=None, help="micro-steps per step (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="no HIP events at all (no roofline, no breakdown)")
    ap.add_argument("--traffic-probe", metavar="SITE", help="one marked micro-step for an HBM counter run")
    ap.add_argument("--counter-probe", action="store_true",
                    help="one micro-step + optimizer step + calibration copy, for per-kernel counter runs")
    ap.add_argument("--workload", choices=sorted(WORKLOADS) + ["lmhead"], default="gpt2",
                    help="gpt2 (the headline step, default), rotary (the modern variant) or lmhead (the isolated "
                         "tied lm_head + cross-entropy)")
    ap.add_argument("--doc-mask", type=float, default=None, metavar="MEAN_DOC",
                    help="packed windows under the document mask, documents of this mean length in tokens "
                         "(default: the plain causal step over documents of mean length 1000)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (--gpus must be 1)",
              file=sys.stderr)
        return 2
    if args.traffic_probe:
        return traffic_probe(args.traffic_probe, args.workload)
    if args.counter_probe:
        return counter_probe(args.workload)
    if args.workload == "lmhead":
        return bench_lmhead(args)

    import numpy as np
    import torch
    import gpt_pretraining_step_amd as g
    import synthetic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = WORKLOADS[args.workload]
    B = wl["B"]
    ga = args.grad_accum if args.grad_accum is not None else wl["G"]
    model = g.GPT2(g.GPT2_124M if args.workload == "gpt2" else g.GPT2_ROTARY_124M)
    model.init_params(seed=42)
    n_params = model.sizes.n_params
    mean_doc = args.doc_mask if args.doc_mask else 1000.0
    stream = synthetic.token_stream(ga * B * T + 1, seed=1337, mean_doc=mean_doc)
    if args.doc_mask:
        model.set_doc_mask(synthetic.EOT_ID)
    xs, ys = [], []
    for k in range(ga):
        x, y = synthetic.micro_batch(stream, k, B, T)
        xs.append(torch.from_numpy(x).cuda())
        ys.append(torch.from_numpy(y).cuda())
    torch.cuda.synchronize()
    losses = torch.zeros(ga, dtype=torch.float32, device="cuda")

    def step():
        model.zero_grad()
        for k in range(ga):
            model.fwd_bwd(xs[k], ys[k], loss_scale=1.0 / ga, loss_out=losses[k:k + 1])
        norm = model.clip_adamw_step(lr=wl["lr"], beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0)
        # the loss is read back once per step, as a logger would
        return float(losses.mean().item()), float(norm.item())

    # Warm-up.  The first warm-up step is also the per-site breakdown: every
    # launch bracketed with events (that adds about 6% to its wall time, so
    # the timed steps below bracket only the dominant kernel).
    fl = gemm_site_flops(B * T, wl["F"], 2 * wl["F"] if args.workload == "rotary" else wl["F"])
    breakdown, gsite = {}, None
    for w in range(max(1, args.warmup)):
        if w == 0 and not args.no_profile:
            model.profile(True)
            model.profile_only(None)
            model.profile_reset()
        step()
        if w == 0 and not args.no_profile:
            st = model.status()
            if st != 0:
                raise RuntimeError(f"device status {st} during warm-up")
            breakdown = model.profile_entries()
            model.profile(False)
            gemm_sites = {k: v for k, v in breakdown.items() if k in fl}
            gsite = max(gemm_sites.items(), key=lambda kv: kv[1][1])[0] if gemm_sites else None
    st = model.status()
    if st != 0:
        raise RuntimeError(f"device status {st} after warm-up")
    print(f"[bench] warm-up done ({max(1, args.warmup)} steps)", file=sys.stderr, flush=True)

    if gsite is not None:
        model.profile(True)
        model.profile_only(gsite)
        model.profile_reset()
    torch.cuda.synchronize()
    step_times, log = [], []
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        for i in range(args.steps):
            s0 = time.perf_counter()
            loss, norm = step()
            step_times.append(time.perf_counter() - s0)
            log.append((loss, norm))
            print(f"[bench] step {i}: loss {loss:.4f} grad-norm {norm:.4f} {step_times[-1] * 1e3:.1f} ms",
                  file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    st = model.status()
    if st != 0:
        raise RuntimeError(f"device status {st} after timed steps")
    prof = model.profile_entries() if gsite is not None else {}
    model.profile(False)
    model.profile_only(None)

    tokens = args.steps * ga * B * T
    tps = tokens / elapsed
    fpt = flops_per_token(n_params)
    result = {
        "metric": wl["metric"],
        "value": round(tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (Zipf token stream, EOT-prefixed documents; random N(0,0.02) init)",
        "config": {"workload": f"{wl['name']}: {ga} x micro-batch B={B} T={T} + clip 1.0 + AdamW lr {wl['lr']:g}"
                               + (f"; packed windows under the document mask, mean document {mean_doc:g} tokens"
                                  if args.doc_mask else ""),
                   "global_batch_tokens": ga * B * T, "micro_batch": B, "seq_len": T, "grad_accum": ga,
                   "vocab": 50304, "parallelism": "none (1 GPU)"},
        "mfu": round(tps * fpt / PEAK_BF16, 4),
        "flops_per_token": fpt,
        "loss_last_step": round(log[-1][0], 5),
        "grad_norm_last_step": round(log[-1][1], 5),
        "clock": clock.summary(),
    }

    # dominant kernel: the GEMM launch site with the largest summed time in the
    # profiled warm-up step; its launches are timed with HIP events on the
    # library's stream during the timed steps
    if gsite is not None and gsite in prof and prof[gsite][0] > 0:
        from gpt_pretraining_step_amd.profiling import load_traffic
        gcnt, gms = prof[gsite]
        gavg = gms / gcnt / 1e3
        result["roofline"] = {
            "kernel": gsite, "bound": "mfma", "achieved": round(fl[gsite] / gavg / 1e12, 2),
            "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
            "frac": round(fl[gsite] / gavg / PEAK_BF16, 4),
            # HBM bytes per launch from the two counter runs recorded under
            # profiles/ (null when none matches this kernel's current sources)
            "traffic": load_traffic(os.path.join(ROOT, "profiles"), gsite, args.workload),
            "avg_launch_us": round(gavg * 1e6, 2), "flops_per_launch": fl[gsite],
            "launches_timed": gcnt,
        }
        total_ms = sum(ms for _, ms in breakdown.values())
        site, (cnt, ms) = max(breakdown.items(), key=lambda kv: kv[1][1])
        result["time_breakdown_ms_per_step"] = {
            k: round(v[1], 3) for k, v in sorted(breakdown.items(), key=lambda kv: -kv[1][1])}
        result["time_breakdown_note"] = "first warm-up step, every launch bracketed with HIP events"
        result["top_site"] = {"site": site, "share": round(ms / total_ms, 4)}
    model.close()
    del model
    torch.cuda.empty_cache()
    if not args.no_profile:
        pk = measured_peak_tflops()
        peak = max(pk.values())
        result["mfu_vs_measured_peak"] = {"mfu": round(tps * fpt / (peak * 1e12), 4), "peak_tflops": peak,
                                          "products": pk, "note": "8192^3 bf16 products on this box"}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(workload=args.workload)
    print(json.dumps(result))
    return 0


def bench_lmhead(args):
    """The isolated tied lm_head + cross-entropy, forward and backward, at
    hidden [65,536 x 768] bf16, vocabulary 50,304, Zipf targets with 10% set
    to ignore_index -1: W untimed calls, then K calls each bracketed by HIP
    events on the stream they run on; the median call."""
    import torch
    import gpt_pretraining_step_amd as g
    import synthetic
    M, C, V = 65536, 768, 50304
    h, w, t = synthetic.lmhead_inputs(M=M, C=C, V=V, ignore_frac=0.1, seed=1337)
    H = torch.from_numpy(h).to(torch.bfloat16).cuda()
    W = torch.from_numpy(w).to(torch.bfloat16).cuda()
    Tg = torch.from_numpy(t).cuda()
    dw = torch.zeros((V, C), dtype=torch.float32, device="cuda")
    scratch = torch.empty(g.lib().gpt2_lmhead_ce_scratch_bytes(M, C, V), dtype=torch.uint8, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    dh = torch.empty_like(H)
    st = torch.cuda.current_stream()

    def call():
        g.lmhead_ce(H, W, Tg, dw, stream=st, scratch=scratch, loss=loss, dhidden=dh)

    # warm-up: at least `warmup` calls and at least 2 s of them, so that the
    # clocks have left their idle state before the timed calls
    w0, nw = time.perf_counter(), 0
    while nw < max(1, args.warmup) or time.perf_counter() - w0 < 2.0:
        call()
        torch.cuda.synchronize()
        nw += 1
    steps = max(args.steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        for a, b in ev:
            a.record(st)
            call()
            b.record(st)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    ts = sorted(a.elapsed_time(b) / 1e3 for a, b in ev)
    med = ts[len(ts) // 2]
    flops = 3 * 2 * M * C * V
    tf = flops / med / 1e12
    print(f"[bench] lmhead: median {med * 1e3:.3f} ms over {steps} calls, loss {float(loss.item()):.5f}",
          file=sys.stderr, flush=True)
    result = {
        "metric": "isolated tied lm_head + cross-entropy fwd+bwd, hidden 65536x768, V=50304, 1 MI355X",
        "value": round(tf, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(med * 1e3, 3), "ms_mean_wall": round(1e3 * elapsed / steps, 3), "warmup_calls": nw,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (hidden N(0,1), weight N(0,0.02^2), Zipf targets, 10% ignored)",
        "config": {"workload": "lmhead_ce: hidden [65536, 768] bf16, weight [50304, 768] bf16, ignore_index -1, "
                               "rows in chunks of 8192", "rows": M, "n_embd": C, "vocab": V,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "gpt2_lmhead_ce (all launches of one call)", "bound": "mfma",
                     "achieved": round(tf, 2), "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                     "frac": round(flops / med / PEAK_BF16, 4), "traffic": None,
                     "avg_launch_us": round(med * 1e6, 2), "flops_per_launch": flops},
        "loss": round(float(loss.item()), 5),
        "clock": clock.summary(),
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = 8192
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        c0 = time.perf_counter()
        oracle.lmhead_ce(h[:rows], w, t[:rows])
        dt = time.perf_counter() - c0
        result["cpu_baseline"] = {"value": round(3 * 2 * rows * C * V / dt / 1e12, 4), "unit": "TFLOP/s",
                                  "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                                  "sample": f"the oracle's lm_head + loss (float32 NumPy) on the first {rows} rows; "
                                            f"{dt:.1f} s"}
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
