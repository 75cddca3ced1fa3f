"""Throughput of the GPT-2 124M training step on one MI355X.

    python bench.py [--gpus 1] [--steps 3] [--warmup 1] [--no-cpu-baseline]
    python bench.py --traffic-probe SITE     (under rocprofv3 --pmc, see below)

One step is the pages' full optimizer step: zero_grad, 32 micro-steps of
B=16 x T=1024 tokens with loss / 32, global-norm clipping at 1.0 and AdamW
(lr 6e-4, betas 0.9/0.95, eps 1e-8, wd 0.1 on 2-D tensors) -- 524,288 tokens
("How I trained my own GPT-2 124M on FineWeb-Edu" sections 8.1 and 9; the
timing protocol of "Making Training Fast on One GPU": warm-up, then timed
full steps with a device synchronisation on both sides, the loss read back
once per step).  Inputs are a synthetic Zipf token stream resident in HBM
before timing starts; weights are the library's own N(0, 0.02) init.

Prints one JSON line with tokens/s, MFU, the roofline of the dominant kernel
(its launches timed with HIP events on the library's stream during the timed
steps; the per-site breakdown comes from the first warm-up step), and the CPU
oracle timed on a bounded sample on this host.  The roofline's `traffic`
(HBM bytes per launch of the dominant kernel) is read from a record under
profiles/ written by `python -m gpt_pretraining_step_amd.profiling traffic`
from two counter runs of `--traffic-probe`, and is null when no record
matches the kernel's current sources.
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


def gemm_site_flops(rows=B * T, F=3072, FC=None, L=12):
    """Algorithmic FLOPs of one launch at each GEMM site of the micro-step
    (rows = B*T, C = 768, MLP width F, V = 50304; the lm_head products take
    all rows in one launch).  FC is the fc product's output width: F for
    GPT-2, 2F (gate and up) for the rotary variant.  gemm.dw is the grouped
    launch of every weight-gradient product: the tied embedding's (lm_head)
    and the L blocks' four each."""
    M, C, V = rows, 768, 50304
    FC = F if FC is None else FC
    return {
        "gemm.dw": 2 * M * V * C + L * 2 * M * C * (3 * C + C + FC + F),
        "gemm.qkv": 2 * M * 3 * C * C,
        "gemm.attn_proj": 2 * M * C * C,
        "gemm.fc": 2 * M * FC * C,
        "gemm.mlp_proj": 2 * M * C * F,
        "gemm.lm_head": 2 * M * V * C,
        "gemm.lm_head_dx": 2 * M * V * C,
        "gemm.lm_head_dw": 2 * M * V * C,
        "gemm.mlp_proj_dw": 2 * M * C * F,
        "gemm.mlp_proj_dx": 2 * M * C * F,
        "gemm.fc_dw": 2 * M * FC * C,
        "gemm.fc_dx": 2 * M * FC * C,
        "gemm.attn_proj_dw": 2 * M * C * C,
        "gemm.attn_proj_dx": 2 * M * C * C,
        "gemm.qkv_dw": 2 * M * 3 * C * C,
        "gemm.qkv_dx": 2 * M * 3 * C * C,
    }


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


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--grad-accum", type=int, default=None, help="micro-steps per step (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="no HIP events at all (no roofline, no breakdown)")
    ap.add_argument("--traffic-probe", metavar="SITE", help="one marked micro-step for an HBM counter run")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="gpt2",
                    help="gpt2 (the headline step, default) or rotary (the modern variant)")
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
    t0 = time.perf_counter()
    step_times, log = [], []
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
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(workload=args.workload)
    model.close()
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
