"""Benchmark of one GPT-2 pre-training step on one MI355X.

A step is the whole hot path: gpt2_accumulate (k micro-batches of forward,
cross-entropy and backward) followed by gpt2_clip_adamw_step, on synthetic
Zipf(1.1) token streams already resident in HBM, with random-init weights of
the GPT-2 small architecture (12 layers, 12 heads, 768 dims, T = 1024,
vocabulary padded to 50,304, tied lm_head), micro-batch 16, accumulation 4,
bf16 compute with fp32 master weights and AdamW moments.

Prints one JSON line: tokens/s (value), MFU against the bf16 dense MFMA peak,
the roofline of the dominant kernel (timed with HIP events inside the timed
region), and the fp64 oracle timed on the host cores as a CPU baseline.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "train tokens/s + MFU (% bf16 MFMA peak), GPT-2 124M T=1024, 1 MI355X"

# Dominant kernel for the roofline object: the launch site whose kernel takes
# the most time per step (from the rocprofv3 kernel trace of this command).
ROOFLINE_SITE = "gemm.fwd.lmhead"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="gpt2-124m")
    ap.add_argument("--site", default=ROOFLINE_SITE, help="launch-site prefix timed for the roofline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="also time every launch site (extra pass)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy (scale reference for HBM byte counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_fwd_lmhead_124m_traffic.md")
TRAFFIC_SOURCE = os.path.join(ROOT, "gpt_decoder_pre_amd", "csrc", "gemm.hip")


def measured_traffic(site):
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None if there is none for this site or
    the kernel source changed since the counters were taken."""
    import hashlib
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
        rec = json.loads(next(l for l in lines if l.startswith("traffic: "))[len("traffic: "):])
        sha = hashlib.sha256(open(TRAFFIC_SOURCE, "rb").read()).hexdigest()
    except (OSError, StopIteration, ValueError):
        return None
    if rec.get("site") != site or rec.get("source_sha256") != sha:
        return None
    return float(rec["bytes_per_launch"])


def flops_per_token(s, T):
    """Algorithmic training FLOPs per token: 6 N + 6 L C T (causal attention),
    N = parameters without wpe; and the 6 N + 12 L C T convention."""
    from gpt2_inputs import n_params
    N = n_params(s) - s.block_size * s.n_embd
    return 6 * N + 6 * s.n_layer * s.n_embd * T, 6 * N + 12 * s.n_layer * s.n_embd * T


def cpu_baseline(run, s):
    """The fp64 oracle as it stands: one full step (forward, backward, clip,
    AdamW) on one sequence of T tokens of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from gpt2_inputs import init_params, micro_batches, token_stream
    from oracle import gpt2 as ref

    T = run.seq_len
    p = init_params(s, run.seed_weights)
    b = micro_batches(token_stream(run.tokens, T + 1, s.vocab_size, run.seed_tokens), 1, 1, T)
    z = {n: np.zeros(a.shape) for n, a in p.items()}
    t0 = time.perf_counter()
    ref.train_step(p, z, z, 1, b, s.n_head, lr=run.lr, weight_decay=run.weight_decay, max_norm=run.max_norm)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(T / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one fp64 oracle step (forward, backward, clip, AdamW) on 1 x {T} tokens of "
                      f"{s.name}, {dt:.1f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the data-parallel split across GPUs "
              f"is not part of this build", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from gpt2_inputs import RUNS, init_params, micro_batches, token_stream
    from gpt_decoder_pre_amd.lib import GPT2Step

    run = RUNS[args.config]
    s = run.shape
    B, T, k = run.micro_batch, run.seq_len, run.grad_accum
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    step = GPT2Step(s, run.precision, max_batch=B, device="cuda:0")
    step.load_params(init_params(s, run.seed_weights))
    # distinct synthetic batches per step, all resident in HBM before timing
    nb = max(1, min(args.steps, 4))
    toks = token_stream(run.tokens, nb * k * B * T + 1, s.vocab_size, run.seed_tokens, run.zipf_s)
    xs, ys = [], []
    for i in range(nb):
        mb = micro_batches(toks[i * k * B * T:(i + 1) * k * B * T + 1], k, B, T)
        xs.append(torch.tensor(np.stack([m[0] for m in mb]), dtype=torch.int32, device=dev))
        ys.append(torch.tensor(np.stack([m[1] for m in mb]), dtype=torch.int32, device=dev))

    def one_step(i):
        step.accumulate(xs[i % nb], ys[i % nb])
        step.clip_adamw_step(run.lr, run.beta1, run.beta2, run.eps, run.weight_decay, run.max_norm)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    if step.sync_status() != 0:
        raise RuntimeError("device error during warm-up")

    step.timing_enable(args.site)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        one_step(i)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop)
    k_ms, k_n, k_flops, k_bytes = step.timing_read()
    step.timing_enable(None)
    loss = float(step.d_loss.item())
    if step.sync_status() != 0 or not np.isfinite(loss):
        raise RuntimeError("device error or non-finite loss in the timed steps")

    tokens = args.steps * k * B * T
    tok_s = tokens / (ms / 1e3)
    f_alg, f_palm = flops_per_token(s, T)
    mfu = tok_s * f_alg / (PEAK_BF16_TFLOPS * 1e12)
    mfu_palm = tok_s * f_palm / (PEAK_BF16_TFLOPS * 1e12)

    roof = None
    if k_n > 0 and k_ms > 0:
        avg_ms = k_ms / k_n
        if k_flops > 0:
            ach = (k_flops / k_n) / (avg_ms / 1e3) / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(args.site)}
            roof["algorithmic_bytes"] = round(k_bytes / k_n)
        else:
            ach = (k_bytes / k_n) / (avg_ms / 1e3) / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
        roof["kernel"] = args.site
        roof["launches"] = int(k_n)
        roof["avg_launch_us"] = round(1e3 * avg_ms, 2)

    breakdown = None
    if args.breakdown:
        breakdown = {}
        for site in ("gemm.fwd", "gemm.bwd", "attn.fwd", "attn.bwd", "ln.fwd", "ln.bwd", "xent", "embed.bwd",
                     "norm", "adamw", "gemm.fwd.qkv", "gemm.fwd.proj", "gemm.fwd.fc", "gemm.fwd.fcproj",
                     "gemm.fwd.lmhead", "gemm.bwd.lmhead.dx", "gemm.bwd.lmhead.dw", "gemm.bwd.fcproj.dx",
                     "gemm.bwd.fcproj.dw", "gemm.bwd.fc.dx", "gemm.bwd.fc.dw", "gemm.bwd.proj.dx", "gemm.bwd.proj.dw",
                     "gemm.bwd.qkv.dx", "gemm.bwd.qkv.dw", "gemm.bwd.dw"):
            step.timing_enable(site)
            one_step(0)
            sm, sn, sf, sb = step.timing_read()
            step.timing_enable(None)
            if sn == 0:  # e.g. per-site weight gradients when they run as one grouped launch
                continue
            breakdown[site] = {"ms_per_step": round(sm, 3), "launches": int(sn),
                               "tflops": round(sf / max(sm, 1e-9) / 1e9, 1) if sf else None,
                               "gbs": round(sb / max(sm, 1e-9) / 1e6, 1)}

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if run.precision == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{s.name} pre-training step: {s.n_layer} layers, {s.n_head} heads, "
                               f"{s.n_embd} dims, vocab {s.padded_vocab_size} (tied), Zipf(1.1) token ids",
                   "micro_batch": B, "grad_accum": k, "seq_len": T, "tokens_per_step": k * B * T,
                   "precision": "bf16 compute, fp32 master weights and AdamW moments"},
        "mfu_pct": round(100 * mfu, 2),
        "mfu_pct_6n_12lct": round(100 * mfu_palm, 2),
        "flops_per_token": f_alg,
        "final_loss": round(loss, 5),
        "roofline": roof,
    }
    if breakdown is not None:
        out["breakdown"] = breakdown
    step.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(run, s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
