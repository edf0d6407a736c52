"""Throughput of the Llama 2 decoder forward on one MI355X: greedy generate at the 7B shape.

One step = one whole greedy generate of the workload (prefill of the prompt batch, then one
single-token decode call per generated position, each followed by the on-device argmax and
token select), with weights, prompts and KV cache already resident in HBM.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--skip-cpu-baseline]

Prints one JSON line.  `value` is decode tokens/s (batch * decode calls / decode time);
prefill tokens/s (batch * prompt_len / prefill time) is reported beside it.  `roofline` is
the dominant decode kernel (the fused RMSNorm + [w1;w3] + SiLU-gate GEMV, about 43% of the
bytes a 7B decode step streams): algorithmic bytes per launch over its average launch
duration, timed live with HIP events bound to each of its dispatches; `traffic` is the HBM
bytes per launch that rocprofv3 counters measured for the same kernel and workload (kept
under profiles/, reported only while the kernel's sources are unchanged).  `cpu_baseline` is the NumPy
oracle on this host's cores over a bounded sample (the whole model, the first decode calls).
`mfma_prefill` times, beside the main line, the MFMA-bound 7B prefill: the 32 ragged prompts of
the batch-32 workload (about 8.4k rows), reported against the dense bf16 MFMA peak.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode tok/s + prefill tok/s, 7B shape, 1 MI355X; % HBM / MFMA roofline"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def decode_step_bytes(wl, ctx: int) -> float:
    """Algorithmic HBM bytes of one decode call at context length ctx (weights once, K/V of
    positions [0, ctx) read, one position written)."""
    D, L, F, V = wl.dim, wl.n_layers, wl.hidden_dim, wl.vocab_size
    hd, H, KVH, B = wl.head_dim, wl.n_heads, wl.n_kv_heads, wl.batch
    e = 4 if wl.dtype == "fp32" else 2
    per_layer = (H * hd * D + 2 * KVH * hd * D + D * H * hd + 3 * F * D + 2 * D) * e
    weights = L * per_layer + V * D * e + D * e + B * D * e
    kv = B * L * 2 * KVH * hd * e * (ctx + 1)
    return weights + kv


def prefill_flops(wl, B: int, S: int, start_pos: int = 0) -> float:
    """Algorithmic flops of a prefill of S tokens per row at start_pos: the projections of
    every row, causal attention (query i sees start_pos + i + 1 keys), the last positions'
    logits."""
    D, L, F, V = wl.dim, wl.n_layers, wl.hidden_dim, wl.vocab_size
    hd, H, KVH = wl.head_dim, wl.n_heads, wl.n_kv_heads
    per_layer = H * hd * D + 2 * KVH * hd * D + D * H * hd + 3 * F * D
    keys = S * start_pos + S * (S + 1) / 2
    return 2.0 * B * S * per_layer * L + 4.0 * hd * H * L * B * keys + 2.0 * B * V * D


def prefill_bytes(wl, B: int, S: int) -> float:
    """Algorithmic HBM bytes of one prefill call: every weight once (embedding: the B*S rows
    read), the K/V of the B*S positions written, the last positions' logits written."""
    D, L, F, V = wl.dim, wl.n_layers, wl.hidden_dim, wl.vocab_size
    hd, H, KVH = wl.head_dim, wl.n_heads, wl.n_kv_heads
    e = 4 if wl.dtype == "fp32" else 2
    per_layer = (H * hd * D + 2 * KVH * hd * D + D * H * hd + 3 * F * D + 2 * D) * e
    return L * per_layer + V * D * e + D * e + B * S * D * e + B * S * L * 2 * KVH * hd * e + B * V * 4


def launch_bytes(kernel_class: str, wl) -> float:
    """Algorithmic HBM bytes of one launch of a decode projection class at the workload's
    batch B: the weight matrices once, plus the activation rows it reads and writes (fp32
    rows on the vector path; the residual products read and write the fp32 residual rows)."""
    e = 4 if wl.dtype == "fp32" else 2
    D, F, V, B = wl.dim, wl.hidden_dim, wl.vocab_size, wl.batch
    nq, nk = wl.n_heads * wl.head_dim, wl.n_kv_heads * wl.head_dim
    if kernel_class == "gemv_qkv":     # fused norm + [wq; wk; wv] + RoPE + q store + K/V append
        return (nq + 2 * nk) * D * e + D * e + B * D * 4 + B * nq * 4 + B * 2 * nk * e
    if kernel_class == "gemv_wo":      # wo + residual add
        return D * nq * e + B * nq * 4 + 2 * B * D * 4
    if kernel_class == "gemv_w13":     # fused norm + [w1; w3] + SiLU gate
        return 2 * F * D * e + D * e + B * D * 4 + B * F * 4
    if kernel_class == "gemv_w2":      # w2 + residual add
        return D * F * e + B * F * 4 + 2 * B * D * 4
    if kernel_class == "gemv_out":     # fused final norm + vocab projection
        return V * D * e + D * e + B * D * 4 + B * V * 4
    raise ValueError(f"no per-launch byte count for kernel class {kernel_class!r}: "
                     "the roofline line takes the decode projection classes gemv_qkv, gemv_wo, "
                     "gemv_w13, gemv_w2, gemv_out")


def mfma_prefill(workload: str, runs: int = 3) -> dict:
    """The MFMA-bound 7B prefill: the prompt batch of `workload` (32 ragged prompts, the
    prefill call covers the shortest prompt of every row, about 8.4k rows), its own seeded
    weights, timed over `runs` calls after one warm-up, with the on-device argmax and select
    as in a generate's first call."""
    import torch
    import synth
    from decoder_only_transformer_amd import runtime
    wl = synth.WORKLOADS[workload]
    W = synth.gen_weights(wl, device="cuda")
    model = runtime.LlamaModel(runtime.make_args(
        wl.dim, wl.n_layers, wl.n_heads, wl.n_kv_heads, wl.vocab_size, wl.hidden_dim,
        wl.norm_eps, wl.rope_theta, wl.batch, wl.max_seq_len, wl.dtype), W)
    run = runtime.GreedyRun(model, synth.prompts(wl), wl.gen_steps, keep_logits=False)
    run.reset()
    run.prefill()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(runs):
        run.reset()
        run.prefill()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / runs
    B, S = run.bsz, run.min_len
    flops = prefill_flops(wl, B, S)
    out = {"workload": wl.name, "batch": B, "prompt_len": S, "rows": B * S, "ms": round(ms, 3),
           "tok_per_s": round(B * S / (ms / 1e3), 1), "tflops": round(flops / (ms / 1e3) / 1e12, 1),
           "mfma_frac": round(flops / (ms / 1e3) / (BF16_PEAK_TFLOPS * 1e12), 4),
           "flops": flops, "runs": runs}
    # Prefill over a cached prefix (the mask's (seqlen, start_pos + seqlen) form): 4 rows of
    # 2048 tokens at start_pos 2048, after a first 2048-token chunk filled the cache, with the
    # same weights; the timed calls rewrite positions [2048, 4096) and read [0, 4096).
    import numpy as np
    cb, cs = 4, 2048
    tok = torch.from_numpy(np.random.Generator(np.random.PCG64(7)).integers(
        3, wl.vocab_size, size=(cb, 2 * cs)).astype(np.int32)).cuda()
    lg = torch.empty((cb, wl.vocab_size), device="cuda")
    model.prefill(tok, cb, cs, 0, lg)
    model.prefill(tok, cb, cs, cs, lg, col=cs)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(runs):
        model.prefill(tok, cb, cs, cs, lg, col=cs)
    ev[1].record()
    torch.cuda.synchronize()
    cms = ev[0].elapsed_time(ev[1]) / runs
    cfl = prefill_flops(wl, cb, cs, cs)
    out["cached_prefix"] = {"batch": cb, "start_pos": cs, "prompt_len": cs, "ms": round(cms, 3),
                            "tok_per_s": round(cb * cs / (cms / 1e3), 1),
                            "tflops": round(cfl / (cms / 1e3) / 1e12, 1),
                            "mfma_frac": round(cfl / (cms / 1e3) / (BF16_PEAK_TFLOPS * 1e12), 4),
                            "flops": cfl}
    model.close()
    del W, run
    torch.cuda.empty_cache()
    return out


def measured_traffic(kernel_class: str, workload: str):
    """HBM bytes per launch of `kernel_class` on `workload` from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads for a
    device copy of known size), or None if there is none or the kernel's sources have
    changed since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"{kernel_class}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        k, sep, v = line.partition(":")
        if sep and k.strip() in ("traffic_bytes_per_launch", "kernel_source_sha256"):
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for name in ("gemv.hip", "common.h", "kernels.h"):
        with open(os.path.join(here, "decoder_only_transformer_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if fields.get("kernel_source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def cpu_baseline(wl, dev_weights, prompts, decode_steps: int = 48, max_fp32_bytes: float = 32e9,
                 max_tokens: int = 4096) -> dict:
    """The oracle as it stands, on this host, over a bounded sample of the same workload.

    Workloads whose fp32 weights fit in `max_fp32_bytes` and whose prompt batch has at most
    `max_tokens` tokens: the whole model (every layer and the head) in fp32 NumPy, prefill of
    the prompt batch and then the first `decode_steps` single-token decode calls; nothing is
    scaled.  Larger ones: the first 2 layers and the head, prefill of at most 1024 prompt
    tokens (the first rows, or the first 1024 tokens of row 0) and 4 decode calls of those rows,
    with the times scaled by n_layers / 2 ("scaled" in the sample description)."""
    import dataclasses
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        threads = max((p.get("num_threads", 1) for p in pools), default=1)
        blas = ",".join(sorted({str(p.get("internal_api", "?")) for p in pools})) or "?"
    except Exception:
        threads, blas = os.cpu_count(), "?"

    cache = {}

    def provider(name, layer):
        k = (name, layer)
        if k not in cache:
            t = dev_weights[name] if layer < 0 else dev_weights["layers"][layer][name]
            cache[k] = t.float().cpu().numpy()
        return cache[k]
    tok = np.array([p[:min(len(x) for x in prompts)] for p in prompts])
    B, S = tok.shape
    e = 4  # the oracle's fp32 copy of every weight
    fp32_bytes = e * (wl.n_layers * (2 * wl.dim * wl.dim + 2 * wl.n_kv_heads * wl.head_dim * wl.dim
                                     + 3 * wl.hidden_dim * wl.dim) + 2 * wl.vocab_size * wl.dim)
    scaled = fp32_bytes > max_fp32_bytes or B * S > max_tokens
    n_layers, scale = wl.n_layers, 1.0
    if scaled:
        rows = max(1, min(B, 1024 // S))
        tok = tok[:rows, :min(S, 1024)]
        B, S = tok.shape
        decode_steps = 4
        n_layers, scale = 2, wl.n_layers / 2.0
    a = dataclasses.replace(oracle.args_from_workload(wl), n_layers=n_layers,
                            max_seq_len=S + decode_steps + 1)
    m = oracle.Oracle(a, provider, B, np.float32)
    m.forward(tok[:, :1], 0)                # first touch: weights to host fp32, BLAS warm-up
    t0 = time.perf_counter()
    logits = m.forward(tok, 0)
    t1 = time.perf_counter()
    nxt = oracle.argmax_lowest(logits[:, -1]).reshape(B, 1)
    for j in range(decode_steps):
        logits = m.forward(nxt, S + j)
        nxt = oracle.argmax_lowest(logits[:, -1]).reshape(B, 1)
    t2 = time.perf_counter()
    what = (f"scaled: the first 2 of {wl.n_layers} layers and the head, times x {scale:g}"
            if scaled else f"all {wl.n_layers} layers and the head")
    return {"value": B * decode_steps / ((t2 - t1) * scale), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "prefill_tok_per_s": B * S / ((t1 - t0) * scale),
            "sample": (f"{wl.name}: oracle fp32 NumPy, {what}, "
                       f"{S}-token prefill of {B} row(s) then {decode_steps} greedy decode calls "
                       f"({t2 - t0:.1f} s timed); host cpu_count={os.cpu_count()}, BLAS {blas} "
                       f"on {threads} threads")}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama2_7b_b1")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--profile-class", default="gemv_w13",
                    choices=["gemv_qkv", "gemv_wo", "gemv_w13", "gemv_w2", "gemv_out"])
    ap.add_argument("--mfma-prefill", default="llama2_7b_b32_ragged",
                    help="workload whose (MFMA-bound) prefill is timed beside the main line; '' skips it")
    ap.add_argument("--gen-steps", type=int, default=0,
                    help="cap on generated positions per step (profiler runs only; 0 = the workload's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import torch
    import synth
    from decoder_only_transformer_amd import abi, runtime

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    abi.lib()
    wl = synth.WORKLOADS[args.workload]
    log(f"[bench] workload {wl}")
    t0 = time.time()
    W = synth.gen_weights(wl, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] weights generated on device in {time.time() - t0:.1f}s")
    prompts = synth.prompts(wl)
    model = runtime.LlamaModel(runtime.make_args(
        wl.dim, wl.n_layers, wl.n_heads, wl.n_kv_heads, wl.vocab_size, wl.hidden_dim,
        wl.norm_eps, wl.rope_theta, wl.batch, wl.max_seq_len, wl.dtype), W)
    gen_steps = min(wl.gen_steps, args.gen_steps) if args.gen_steps > 0 else wl.gen_steps
    run = runtime.GreedyRun(model, prompts, gen_steps, keep_logits=False)
    B, S, n_dec = run.bsz, run.min_len, run.n_calls - 1

    def one_step(ev=None):
        run.reset()
        if ev:
            ev[0].record()
        run.prefill()
        if ev:
            ev[1].record()
        for i in range(1, run.n_calls):
            run.decode(i)
        if ev:
            ev[2].record()

    for w in range(args.warmup):
        one_step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {w + 1}/{args.warmup} done")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        one_step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in evs)
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs)
    log(f"[bench] timed {args.steps} steps: wall {wall:.3f}s prefill {pre_ms / args.steps:.3f} ms/step "
        f"decode {dec_ms / args.steps:.3f} ms/step")
    decode_tps = B * n_dec * args.steps / (dec_ms / 1e3)
    prefill_tps = B * S * args.steps / (pre_ms / 1e3)
    dec_bytes = sum(decode_step_bytes(wl, S + i) for i in range(n_dec))
    decode_hbm_frac = dec_bytes * args.steps / (dec_ms / 1e3) / (HBM_PEAK_GBS * 1e9)
    pf = prefill_flops(wl, B, S)
    prefill_tflops = pf * args.steps / (pre_ms / 1e3) / 1e12

    # Live per-kernel timing of the dominant decode kernel, same launch configuration: one
    # more step, with the class selected after its prefill (the vector path of fp32 / fp16
    # models runs the prefill on the same kernel class, with many rows per launch)
    kc = abi.KERNEL_CLASSES[args.profile_class]
    run.reset()
    run.prefill()
    torch.cuda.synchronize()
    runtime.check("profile_select", abi.llama_profile_select(model.ctx, kc))
    for i in range(1, run.n_calls):
        run.decode(i)
    torch.cuda.synchronize()
    st, n_launch, k_ms = abi.llama_profile_read(model.ctx)
    runtime.check("profile_read", st)
    abi.llama_profile_select(model.ctx, 0)
    avg_us = k_ms / max(n_launch, 1) * 1e3
    per_launch = launch_bytes(args.profile_class, wl)
    achieved = per_launch / (avg_us * 1e-6) / 1e9
    log(f"[bench] {args.profile_class}: {n_launch} launches, avg {avg_us:.2f} us, "
        f"{per_launch / 1e6:.1f} MB/launch -> {achieved:.0f} GB/s")

    # Plain device copy for context (bandwidth the HBM actually gives a trivial kernel).
    buf = torch.empty(2 * 1024 ** 3, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(buf)
    dst.copy_(buf)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(buf)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * buf.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    del buf, dst

    mfma = None
    if args.mfma_prefill and args.mfma_prefill != wl.name:
        log(f"[bench] MFMA-bound prefill of {args.mfma_prefill} ...")
        mfma = mfma_prefill(args.mfma_prefill)
        log(f"[bench] {mfma}")

    cpu = None
    if not args.skip_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        t0 = time.time()
        cpu = cpu_baseline(wl, W, prompts)
        log(f"[bench] cpu baseline done in {time.time() - t0:.1f}s")

    out = {
        "metric": METRIC,
        "value": round(decode_tps, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((pre_ms + dec_ms) / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: seeded N(0,0.02) weights, uniform random prompt ids",
        "config": {"workload": wl.name, "batch": B, "prompt_len": S, "decode_calls": n_dec,
                   "dim": wl.dim, "n_layers": wl.n_layers, "n_heads": wl.n_heads,
                   "n_kv_heads": wl.n_kv_heads, "hidden_dim": wl.hidden_dim, "vocab": wl.vocab_size},
        "decode_tok_per_s": round(decode_tps, 2),
        "prefill_tok_per_s": round(prefill_tps, 1),
        "decode_ms_per_call": round(dec_ms / args.steps / n_dec, 4),
        "prefill_ms": round(pre_ms / args.steps, 3),
        "decode_hbm_frac": round(decode_hbm_frac, 4),
        "prefill_tflops": round(prefill_tflops, 2),
        "prefill_mfma_frac": round(prefill_tflops / BF16_PEAK_TFLOPS, 4),
        "prefill_hbm_frac": round(prefill_bytes(wl, B, S) * args.steps / (pre_ms / 1e3) / (HBM_PEAK_GBS * 1e9), 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.profile_class, wl.name),
                     "kernel": args.profile_class, "launches": n_launch, "avg_us": round(avg_us, 3),
                     "bytes_per_launch": per_launch},
        "copy_kernel_gbs": round(copy_gbs, 1),
        "mfma_prefill": mfma,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    model.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
