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
import dataclasses
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

# Launch sites of one step (gpt2_timing_site names them); the roofline object
# describes the one that takes the most time per step, ranked from a
# per-site HIP-event record of one untimed step of this run.


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="gpt2-124m")
    ap.add_argument("--precision", default=None, choices=["fp32", "bf16", "fp16"],
                    help="override the config's precision (fp16: IEEE half operands with dynamic loss scaling)")
    ap.add_argument("--site", default=None, help="launch site timed for the roofline (default: the one that "
                    "takes the most time per step in a per-site record of one untimed step)")
    ap.add_argument("--cpu-toy", action="store_true", help="also time the oracle on the toy step")
    ap.add_argument("--decode", action="store_true",
                    help="instead of the training step, time cached decoding (prefill, then one token per "
                         "sequence per step with top-k / top-p sampling) and print its own JSON line")
    ap.add_argument("--prompt", type=int, default=128, help="prompt length for --decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="instead of the training step, time plain HBM streams (read only, write only, copy, "
                         "add) of 1 GiB fp32 buffers with PyTorch's own kernels and print their rates")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy (scale reference for HBM byte counters)")
    return ap.parse_args()


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gpt_decoder_pre_amd", "csrc")


def measured_traffic(site):
    """HBM bytes per launch of a launch site's kernel from a committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (a `traffic: {json}` line in
    profiles/*_traffic.md), or None if there is none for this site or the
    kernel source it names changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_traffic.md"))):
        try:
            lines = open(path).read().splitlines()
            rec = json.loads(next(l for l in lines if l.startswith("traffic: "))[len("traffic: "):])
            if rec.get("site") != site:
                continue
            sha = hashlib.sha256(open(os.path.join(CSRC, rec["source"]), "rb").read()).hexdigest()
        except (OSError, StopIteration, ValueError, KeyError):
            continue
        if rec.get("source_sha256") == sha:
            return float(rec["bytes_per_launch"])
    return None


def site_roofline(ms, n, flops, bytes_):
    """Achieved rate of a site's launches against the MI355X peak that bounds
    it: dense bf16 MFMA for products, HBM for the streaming kernels."""
    avg_ms = ms / n
    if flops > 0:
        ach = (flops / n) / (avg_ms / 1e3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    ach = (bytes_ / n) / (avg_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4)}


def flops_per_token(s, T):
    """Algorithmic training FLOPs per token: 6 N + 6 L C T (causal attention),
    N = parameters without wpe; and the 6 N + 12 L C T convention."""
    from gpt2_inputs import n_params
    # wpe (and wte when the head is its own tensor) is a gather, not a product
    N = n_params(s) - s.block_size * s.n_embd - (0 if s.tied else s.padded_vocab_size * s.n_embd)
    return 6 * N + 6 * s.n_layer * s.n_embd * T, 6 * N + 12 * s.n_layer * s.n_embd * T


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(run, s, toy=False):
    """The fp64 oracle as it stands: one full step (forward, backward, clip,
    AdamW) on one sequence of T tokens of the same workload (and, with toy,
    the whole char-level toy step)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from gpt2_inputs import RUNS, init_params, micro_batches, token_stream
    from oracle import gpt2 as ref

    def one(r, shape, B, T, k):
        p = init_params(shape, r.seed_weights)
        b = micro_batches(token_stream(r.tokens, k * B * T + 1, shape.vocab_size, r.seed_tokens), k, B, T)
        z = {n: np.zeros(a.shape) for n, a in p.items()}
        t0 = time.perf_counter()
        ref.train_step(p, z, z, 1, b, shape.n_head, lr=r.lr, weight_decay=r.weight_decay, max_norm=r.max_norm)
        return time.perf_counter() - t0

    T = run.seq_len
    dt = one(run, s, 1, T, 1)
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info if i.get("user_api") == "blas"}))
    out = {"value": round(T / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"one fp64 oracle step (forward, backward, clip, AdamW) on 1 x {T} tokens of "
                     f"{s.name}, {dt:.1f} s wall",
           "cpu_model": _cpu_model(), "blas": blas or "unknown",
           "affinity_cpus": len(os.sched_getaffinity(0))}
    if toy:
        tr = RUNS["toy"]
        dtt = one(tr, tr.shape, tr.micro_batch, tr.seq_len, tr.grad_accum)
        out["toy"] = {"value": round(tr.tokens_per_step / dtt, 1), "unit": "tokens/s",
                      "sample": f"the whole toy step ({tr.micro_batch} x {tr.seq_len} tokens, fp64), "
                                f"{dtt * 1e3:.0f} ms wall"}
    return out


def decode_bench(args):
    """Cached decoding of the micro-batch's sequences: per step one token per
    sequence (lm_head logits, the sampler, then the next decode).  A decoding
    step streams every weight once plus the cached keys and values, so its
    roofline is HBM bandwidth."""
    import numpy as np
    import torch

    from gpt2_inputs import RUNS, init_params, token_stream
    from gpt_decoder_pre_amd.lib import Decoder, GPT2Step

    run = RUNS[args.config]
    s = run.shape
    B, T0, n = run.micro_batch, args.prompt, args.steps
    if T0 + args.warmup + n > s.block_size:
        raise SystemExit("--prompt + --warmup + --steps exceeds the block size")
    dev = torch.device("cuda:0")
    st = GPT2Step(s, run.precision, max_batch=1, device="cuda:0")
    st.load_params(init_params(s, run.seed_weights))
    dec = Decoder(st, B)
    prompt = torch.tensor(token_stream("zipf", B * T0, s.vocab_size, run.seed_tokens).reshape(B, T0),
                          dtype=torch.int32, device=dev)
    u = torch.rand((args.warmup + n, B), generator=torch.Generator(device=dev).manual_seed(1), device=dev)
    z = dec.prefill(prompt)
    for i in range(args.warmup):
        z = dec.decode(dec.sample(z, u[i], 0.8, 40, 0.95))
    torch.cuda.synchronize()
    len0 = dec.length()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(n):
        z = dec.decode(dec.sample(z, u[args.warmup + i], 0.8, 40, 0.95))
    t1.record()
    torch.cuda.synchronize()
    if dec.sync_status() != 0:
        raise RuntimeError("device error in decoding")
    ms = t0.elapsed_time(t1) / n
    from gpt2_inputs import n_params
    w_bytes = 2 * (n_params(s) - s.block_size * s.n_embd)  # bf16 weights, each read once per step
    kv = 2 * s.n_layer * B * (len0 + n / 2) * 2 * s.n_embd  # cached keys and values, mean length
    byt = w_bytes + kv + 4 * B * s.padded_vocab_size
    ach = byt / (ms / 1e3) / 1e9
    out = {"metric": "decode tokens/s (cached, one token per sequence per step, top-k 40 / top-p 0.95)",
           "value": round(B / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
           "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{s.name} decoding, {B} sequences, prompt {T0}, positions {len0}..{len0 + n}"},
           "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(ach / PEAK_HBM_GBS, 4), "algorithmic_per_step": int(byt),
                        "algorithmic_unit": "byte", "traffic": None}}
    dec.close()
    st.close()
    print(json.dumps(out), flush=True)


def hbm_ceiling_bench(args):
    """What this part sustains for plain streams, as a reference for the
    HBM-bound kernels of the step: the library's stream probes (read only,
    write only, copy) and PyTorch's own reduction, fill, copy and add kernels
    over 1 GiB fp32 buffers (4x the last-level cache), each timed with HIP
    events on torch's stream over `steps` back-to-back calls after `warmup`
    untimed ones.  Rates are the bytes each op must move (read + written)
    over its time."""
    import torch

    from gpt_decoder_pre_amd import lib as L
    dev = torch.device("cuda:0")
    n = 1 << 28  # 1 GiB of fp32
    g = torch.Generator(device=dev).manual_seed(3)
    x = torch.rand(n, generator=g, device=dev)
    x2 = torch.rand(n, generator=g, device=dev)
    y = torch.empty_like(x)
    acc = torch.empty((), device=dev)
    part = torch.empty(L.probe_partials(n), device=dev)
    nb = 4 * n
    ops = [("probe: read only", lambda: L.stream_probe(L.PROBE_READ, x, part), nb),
           ("probe: write only", lambda: L.stream_probe(L.PROBE_WRITE, None, y), nb),
           ("probe: copy", lambda: L.stream_probe(L.PROBE_COPY, x, y), 2 * nb),
           ("torch: read only (sum)", lambda: torch.sum(x, dim=0, out=acc), nb),
           ("torch: write only (fill)", lambda: y.fill_(0.5), nb),
           ("torch: copy (one read, one write)", lambda: y.copy_(x), 2 * nb),
           ("torch: add (two reads, one write)", lambda: torch.add(x, x2, out=y), 3 * nb)]
    steps, warm = max(args.steps, 10), max(args.warmup, 3)
    rows = []
    for name, fn, byt in ops:
        for _ in range(warm):
            fn()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / steps
        if name == "probe: read only":  # the partial sums add up to the buffer's sum
            want = float(torch.sum(x.double()))
            got = float(torch.sum(part.double()))
            if abs(got - want) > 1e-3 * abs(want):
                raise RuntimeError(f"read probe sum {got} != {want}")
        if name == "probe: write only" and not bool((y == 0.5).all()):
            raise RuntimeError("write probe result")
        if name == "probe: copy" and not torch.equal(y, x):
            raise RuntimeError("copy probe result")
        gbs = byt / (us * 1e-6) / 1e9
        rows.append({"stream": name, "bytes": byt, "us": round(us, 1), "GB/s": round(gbs, 1),
                     "frac": round(gbs / PEAK_HBM_GBS, 4)})
    if not torch.equal(y, x + x2):
        raise RuntimeError("add stream result")
    print(json.dumps({"metric": "HBM stream rates of plain kernels (1 GiB fp32 buffers)", "unit": "GB/s",
                      "peak": PEAK_HBM_GBS, "steps": steps, "warmup": warm, "rows": rows}), flush=True)


def main():
    args = parse()
    if args.hbm_ceiling:
        hbm_ceiling_bench(args)
        return
    if args.decode:
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        decode_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the data-parallel split across GPUs "
              f"is not part of this build", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from gpt2_inputs import RUNS, init_params, micro_batches, token_stream
    from gpt_decoder_pre_amd.lib import GPT2Step

    run = RUNS[args.config]
    if args.precision:
        run = dataclasses.replace(run, precision=args.precision)
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

    # per-site record of one untimed step: ranks the sites by time per step
    step.timing_enable("")
    one_step(0)
    sites = sorted(step.timing_sites(), key=lambda r: -r["ms"])
    step.timing_enable(None)
    site = args.site or sites[0]["site"]
    step_ms = sum(r["ms"] for r in sites)
    breakdown = []
    for r in sites[:12]:
        e = {"site": r["site"], "ms_per_step": round(r["ms"], 3), "share": round(r["ms"] / step_ms, 4),
             "launches": r["launches"], "gemm_cfg": r["gemm_cfg"]}
        e.update(site_roofline(r["ms"], r["launches"], r["flops"], r["bytes"]))
        breakdown.append(e)

    step.timing_enable(site)
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
        roof = site_roofline(k_ms, k_n, k_flops, k_bytes)
        roof["traffic"] = measured_traffic(site)
        roof["kernel"] = site
        roof["launches"] = int(k_n)
        roof["avg_launch_us"] = round(1e3 * k_ms / k_n, 2)
        roof["algorithmic_per_launch"] = (round(k_flops / k_n) if k_flops > 0 else round(k_bytes / k_n))
        roof["algorithmic_unit"] = "flop" if k_flops > 0 else "byte"

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
        "dtype": {"bf16": "bf16", "fp16": "f16"}.get(run.precision, "f32"),
        "data": "synthetic",
        "config": {"workload": f"{s.name} pre-training step: {s.n_layer} layers, {s.n_head} heads, "
                               f"{s.n_embd} dims, vocab {s.padded_vocab_size} "
                               f"({'tied' if s.tied else 'untied head, no QKV bias'}), Zipf(1.1) token ids",
                   "micro_batch": B, "grad_accum": k, "seq_len": T, "tokens_per_step": k * B * T,
                   "precision": {"bf16": "bf16 compute, fp32 master weights and AdamW moments",
                                 "fp16": "fp16 compute with dynamic loss scaling, fp32 master weights and AdamW "
                                         "moments"}.get(run.precision, "fp32")},
        "mfu_pct": round(100 * mfu, 2),
        "mfu_pct_6n_12lct": round(100 * mfu_palm, 2),
        "flops_per_token": f_alg,
        "final_loss": round(loss, 5),
        "roofline": roof,
        "breakdown": breakdown,
    }
    step.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(run, s, toy=args.cpu_toy or args.config == "gpt2-124m")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
