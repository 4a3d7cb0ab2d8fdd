"""Throughput of the nanochat GPT forward+backward step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d12]
                    [--fp8 auto|on|off] [--no-cpu-baseline] [--roofline-kernel K]
                    [--smear] [--backout]
    python bench.py --decode [--steps K] [--warmup W]
    python bench.py --optimizer [--steps K] [--warmup W]

One step = one gpt_fwd_bwd call (loss + every parameter gradient) over one
batch of seeded synthetic tokens, inputs already resident in HBM. Prints one
JSON line with tokens/s, the model-FLOP fraction of the dense bf16 MFMA peak,
the roofline figures of the dominant kernel (timed with HIP events on the
call's stream during the timed steps) and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402

PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA (published)
PEAK_FP8_FLOPS = 5.0e15       # MI355X dense fp8 MFMA (published)
PEAK_HBM_BYTES = 8.0e12       # MI355X HBM3E (published)
METRIC = "train tokens/sec (fwd+bwd) d12 seq2048, 1 GPU; MFMA util vs bf16 peak"


def _full(l, L):
    return l % 4 == 3 or l == L - 1


def _ve(l, L):
    return (l % 2) == ((L - 1) % 2)


def model_flops_per_token(w) -> float:
    """6 FLOPs per matrix weight used in a product (forward 2, backward 4)
    plus 12 * H * D per visible key per layer (useful attention only; the
    window and the causal mask are not counted)."""
    C, H, Hk, D, F, V, L = (w.n_embd, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden,
                            w.vocab, w.n_layer)
    T, Wn = w.seq_len, w.short_window
    n_mat = V * C + (C if w.smear else 0)
    kbar = 0.0
    for l in range(L):
        n_mat += (H + 2 * Hk) * D * C + C * H * D + 2 * F * C
        if _ve(l, L):
            n_mat += Hk * C
        if _full(l, L):
            kbar += (T + 1) / 2
        else:
            win = min(Wn, T - 1)
            kbar += (win * (win + 1) / 2 + (T - win) * (win + 1)) / T
    return 6.0 * n_mat + 12.0 * H * D * kbar


# Kernels the roofline figure can be taken for: the launch sites that run
# it (timed with HIP events on the call's stream) and the algorithmic FLOPs
# (MFMA-bound) or HBM bytes (bandwidth-bound) of those launches in one step.
def _wgrad_flops(w):
    N = w.batch * w.seq_len
    C, Cq, Qkv, F = (w.n_embd, w.n_head * w.head_dim,
                     (w.n_head + 2 * w.n_kv_head) * w.head_dim, w.mlp_hidden)
    return w.n_layer * 2.0 * N * (Qkv * C + 2 * F * C + C * Cq)


def _block_linear_flops(w):
    """The six block linears' forward, input-gradient and weight-gradient
    products of one step (2 FLOPs per multiply-add, 3 products each)."""
    N = w.batch * w.seq_len
    C, Cq, Qkv, F = (w.n_embd, w.n_head * w.head_dim,
                     (w.n_head + 2 * w.n_kv_head) * w.head_dim, w.mlp_hidden)
    return w.n_layer * 3 * 2.0 * N * (Qkv * C + 2 * F * C + C * Cq)


_BLOCK_SITES = ",".join(f"gemm.{m}.{k}" for m in ("qkv", "o", "fc", "mp")
                        for k in ("fwd", "dgrad", "wgrad"))

ROOF_KERNELS = {
    "wgrad": dict(
        sites="gemm.qkv.wgrad,gemm.fc.wgrad,gemm.mp.wgrad,gemm.o.wgrad",
        desc="weight-gradient GEMMs of the blocks, split-K partial sums (their reduction, "
             "splitk_reduce_kernel, is timed apart): gemm_kmaj_kernel<256, EpPart, 0, NoDeq, true> "
             "(token-major operands, direct LDS fills, 8 wavefronts; the 768 x 768 o-proj gradient "
             "as gemm_kmaj_kernel<128, EpPart, 0, NoDeq, true>); with fp8 block linears gemm_kmaj_kernel<BN, EpPart, 2, Deq8> "
             "on the transposed e5m2 / e4m3 codes",
        flops=_wgrad_flops, pmc="profiles/gemm_wgrad_d12_pmc.txt", fp8_peak=True),
    # every product of the block linears (with fp8 linears: the fp8 MFMA
    # products, against the fp8 peak; their quantisation is timed apart)
    "block_gemm": dict(
        sites=_BLOCK_SITES, desc="the block linears' products (forward, input gradient, weight "
                                 "gradient; split-K sums timed apart)",
        flops=_block_linear_flops, pmc=None, fp8_peak=True),
    "lm_fwd": dict(
        sites="gemm.lm.fwd", desc="lm_head GEMM + tanh softcap epilogue",
        flops=lambda w: 2.0 * w.batch * w.seq_len * w.vocab * w.n_embd, pmc=None),
    # the embedding gather (with --smear: the fused smear, which reads the
    # current and the previous token's rows and writes the mixed row)
    "embed_fwd": dict(
        sites="embed.fwd", bound="hbm",
        desc="embedding gather (smear_embed_kernel with --smear, else embed_kernel)",
        bytes=lambda w: (12.0 if w.smear else 8.0) * w.n_embd * w.batch * w.seq_len, pmc=None),
}


def param_total(w) -> int:
    C, H, Hk, D, F, V, L = (w.n_embd, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden,
                            w.vocab, w.n_layer)
    n = 2 * V * C + 2 * L + (C if w.smear else 0) + (1 if w.backout else 0)
    for l in range(L):
        n += (H + 2 * Hk) * D * C + C * H * D + 2 * F * C
        if _ve(l, L):
            n += V * Hk * D + Hk * C
    return n


def _cpu_cores() -> int:
    """Threads of the host's BLAS pool (what the oracle's NumPy products use)."""
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        return int(max((i.get("num_threads", 0) for i in info), default=os.cpu_count()))
    except Exception:  # pragma: no cover
        return int(os.cpu_count())


def cpu_baseline(w, params, tokens, targets, rows: int):
    """The oracle (unchanged) on the first `rows` batch rows of the same
    inputs: tokens/s of its fwd+bwd, on the host's cores."""
    import oracle  # test infrastructure: only this leg of the benchmark uses it
    sub = w.with_(batch=rows)
    t0 = time.perf_counter()
    oracle.forward_backward(sub, params, tokens[:rows], targets[:rows], dtype=np.float32)
    dt = time.perf_counter() - t0
    return {"value": rows * w.seq_len / dt, "unit": "tokens/s", "cores": _cpu_cores(),
            "kind": "oracle",
            "sample": f"{rows} of {w.batch} batch rows ({rows * w.seq_len} tokens) of the "
                      f"{w.name} workload, one fp32 forward+backward, {dt:.1f} s"}


def decode_bench(args):
    """KV-cache decode attention of the d12 model: one step = the attention
    of all 12 layers for one new token in each of 16 sequences whose caches
    hold 2048 positions (short-window layers read the last 513 positions,
    the full layers all 2048). Each layer has its own cache, so the step
    reads 1.2 GB from HBM rather than from the memory-side cache."""
    import torch
    from decoder_only_pretraining_amd import binding as B
    w = W.get("d12")
    Bs, H, Hk, D, T, L = 16, w.n_head, w.n_kv_head, w.head_dim, w.seq_len, w.n_layer
    g = torch.Generator(device="cuda:0").manual_seed(5)
    dev = "cuda:0"
    wins = [-1 if _full(l, L) else w.short_window for l in range(L)]
    q = [torch.randn(Bs, H, D, device=dev, generator=g).to(torch.bfloat16) for _ in range(L)]
    kc = [torch.randn(Bs, T, Hk, D, device=dev, generator=g).to(torch.bfloat16) for _ in range(L)]
    vc = [torch.randn(Bs, T, Hk, D, device=dev, generator=g).to(torch.bfloat16) for _ in range(L)]
    out = [torch.empty_like(x) for x in q]
    seqlen = torch.full((Bs,), T, dtype=torch.int32, device=dev)
    ws = torch.zeros(max(B.decode_attn_workspace(Bs, H, Hk, D, T, wn) for wn in wins),
                     dtype=torch.uint8, device=dev)  # chunk states, written before read

    def step():
        stream = torch.cuda.current_stream()
        for l in range(L):
            B.decode_attn(q[l], kc[l], vc[l], seqlen, out[l], ws, wins[l], stream)

    # the 24 launches of a step are captured once into a HIP graph, so the
    # timing sees the kernels rather than the host's per-call overhead; the
    # replays must reproduce the eager outputs bit for bit
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in out]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    assert all(torch.equal(e, o) for e, o in zip(eager, out)), "graph replay differs from eager"
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    assert all(torch.equal(e, o) for e, o in zip(eager, out)), "graph replay differs from eager"
    ms = a.elapsed_time(b) / args.steps
    # algorithmic bytes: visible K and V rows, q read, out written
    kv = sum(Bs * Hk * (T if wn < 0 else min(T, wn + 1)) * D * 2 * 2 for wn in wins)
    nbytes = kv + L * 2 * Bs * H * D * 2
    gbs = nbytes / (ms / 1e3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:  # the oracle on the same inputs, all 12 layers
        import oracle  # test infrastructure: only the CPU-baseline legs use it
        host = [(x.float().cpu().numpy(), y.float().cpu().numpy(), z.float().cpu().numpy())
                for x, y, z in zip(q, kc, vc)]
        sl = seqlen.cpu().numpy()
        t0 = time.perf_counter()
        for (qh, kh, vh), wn in zip(host, wins):
            oracle.decode.decode_attention(qh, kh, vh, sl, None if wn < 0 else wn)
        dt = time.perf_counter() - t0
        cpu = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": _cpu_cores(),
               "kind": "oracle", "sample": f"the whole step (12 layers, {Bs} sequences), float64 "
                                           f"NumPy, {dt:.2f} s"}
    print(json.dumps({
        "metric": "KV-cache decode attention read rate, d12 (12 layers), 16 sequences x 2048 "
                  "cached positions", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) q and caches)",
        "config": {"workload": "d12 decode attention: 16 sequences, 2048 cached positions, "
                               "heads 6/6, head_dim 128, 9 window-512 layers + 3 full",
                   "tokens_per_step": Bs},
        "decode_tokens_per_s_attention_only": round(Bs / (ms / 1e3), 1),
        "roofline": {"kernel": "decode_attn_kernel<128, 1, 4> (chunks of 128 cached positions) "
                               "+ decode_attn_combine_kernel<128>",
                     "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_BYTES / 1e9,
                     "unit": "GB/s", "frac": round(gbs / (PEAK_HBM_BYTES / 1e9), 4),
                     "traffic": None, "launches": 2 * L * args.steps,
                     "algorithmic_bytes_per_step": nbytes},
        "cpu_baseline": cpu}), flush=True)


def optimizer_bench(args):
    """The full d12 training step of the pages: 4 accumulated fwd+bwd calls
    of 16,384 tokens (65,536 tokens) and one MuonAdamW step (default
    hyper-parameters of the library's oracle description: the pages' rates,
    5 Newton-Schulz steps); also the optimizer step alone."""
    import torch
    from decoder_only_pretraining_amd import binding as B
    w = W.get("d12")
    total = param_total(w)
    params = W.gen_params(total, w.n_layer, W.weight_seed(w))
    tokens, targets = W.split_tokens(W.gen_tokens(w))
    step = B.Step(w, params, tokens, targets, flags=B.GPT_F_ACCUMULATE, device="cuda:0")
    state = torch.zeros(2 * total, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(B.optim_workspace_size(step.cfg), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()

    def hp(t):
        return B.OptimHparams(step=t, ns_steps=5, nesterov=1, lr_matrix=0.02, lr_scalar=0.5,
                              lr_embed=0.3, lr_unembed=0.008, lr_mult=1.0, weight_decay=0.28,
                              beta1=0.9, beta2=0.999, eps=1e-8, momentum=0.95, ns_a=3.4445,
                              ns_b=-4.7750, ns_c=2.0315)

    t = 0
    # micro-batches 2-4 see the same weights: they keep the bf16 weight
    # mirrors the first call converted
    reuse = B.make_config(w, B.GPT_F_ACCUMULATE | B.GPT_F_REUSE_WEIGHTS)

    def full_step():
        nonlocal t
        t += 1
        step.grads.zero_()
        step.run(stream)
        for _ in range(3):
            B.fwd_bwd(reuse, step.params, step.tokens, step.targets, step.loss, step.grads,
                      step.workspace, stream)
        B.optimizer_step(step.cfg, hp(t), step.params, step.grads, state, ws, stream)

    for _ in range(args.warmup):
        full_step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record(stream)
    for _ in range(args.steps):
        full_step()
    ev[1].record(stream)
    ev[2].record(stream)
    for _ in range(args.optimizer_alone_steps):
        t += 1
        B.optimizer_step(step.cfg, hp(t), step.params, step.grads, state, ws, stream)
    ev[3].record(stream)
    torch.cuda.synchronize()
    full_ms = ev[0].elapsed_time(ev[1]) / args.steps
    opt_ms = (ev[2].elapsed_time(ev[3]) / args.optimizer_alone_steps
              if args.optimizer_alone_steps else None)
    loss = float(step.loss.item())
    assert np.isfinite(loss), loss
    ntok = 4 * w.batch * w.seq_len
    print(json.dumps({
        "metric": "full training step tokens/sec (4 x 16,384-token fwd+bwd + MuonAdamW), d12 "
                  "seq2048, 1 GPU", "value": round(ntok / (full_ms / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(full_ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Zipf(1.1) tokens, N(0,0.02) weights)",
        "config": {"workload": "d12, 65,536 tokens per optimizer step (4 accumulated calls)",
                   "tokens_per_step": ntok},
        "optimizer_ms": None if opt_ms is None else round(opt_ms, 3),
        "context": {"pages_rtx4070_full_step_ms": 1177}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="d12")
    ap.add_argument("--fp8", default="auto", choices=["auto", "on", "off"],
                    help="block linears in fp8 (auto: as the workload defines)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="enqueue every launch of each call (default: the call's launch sequence "
                         "is captured once into a HIP graph and replayed, GPT_F_GRAPH)")
    ap.add_argument("--smear", action="store_true", help="the Smear model variant")
    ap.add_argument("--optimizer", action="store_true",
                    help="time the full step with MuonAdamW (4 accumulated calls + optimizer)")
    ap.add_argument("--optimizer-alone-steps", type=int, default=10,
                    help="with --optimizer: optimizer steps timed on their own after the full steps")
    ap.add_argument("--decode", action="store_true",
                    help="time the KV-cache decode attention instead of the training step")
    ap.add_argument("--backout", action="store_true",
                    help="the Backout model variant (lambda 0.5)")
    ap.add_argument("--cpu-rows", type=int, default=3)
    ap.add_argument("--roofline-kernel", default="wgrad", choices=sorted(ROOF_KERNELS),
                    help="kernel whose launches are timed with HIP events for the roofline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU path is "
              "not part of this library", file=sys.stderr)
        sys.exit(2)

    if args.decode:
        decode_bench(args)
        return
    if args.optimizer:
        optimizer_bench(args)
        return

    import torch
    from decoder_only_pretraining_amd import binding as B

    w = W.get(args.config)
    if args.fp8 != "auto":
        w = w.with_(fp8_linears=args.fp8 == "on")
    w = w.with_(smear=args.smear, backout=args.backout)
    total = param_total(w)
    params = W.gen_params(total, w.n_layer, W.weight_seed(w))
    if w.backout:  # the additions page's table: Backout subtracts half
        lay = {n: o for n, o, _, _ in B.param_layout(B.make_config(w))}
        params[lay["backout_lambda"]] = 0.5
    tokens, targets = W.split_tokens(W.gen_tokens(w))
    graph = not args.no_graph
    step = B.Step(w, params, tokens, targets, flags=B.GPT_F_GRAPH if graph else 0,
                  device="cuda:0")
    # a stream of its own (a HIP graph cannot be captured on the null stream),
    # after the uploads on the default stream have finished
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    roof_k = ROOF_KERNELS[args.roofline_kernel]
    for _ in range(args.warmup):   # with the graph: the first call captures it
        step.run(stream)
    torch.cuda.synchronize()
    # eager launches: the dominant kernel's launches are bracketed by HIP
    # events on the call's stream inside the timed region; with the graph
    # they are timed the same way over eager steps right after it (same
    # buffers and stream; a kernel's duration does not depend on how it was
    # enqueued)
    if not graph:
        B.profile_begin(roof_k["sites"])

    # one event before every step and one after the last, on the step's
    # stream: the whole timed region and each step's time
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i].record(stream)
        step.run(stream)
    ev[args.steps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev[0].elapsed_time(ev[args.steps])
    steps_timed = args.steps if not graph else min(args.steps, 10)
    if graph:
        B.profile_begin(roof_k["sites"])
        for _ in range(steps_timed):
            step.run(stream)
    kern_ms, kern_n = B.profile_end()
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    loss = float(step.loss.item())
    assert np.isfinite(loss), loss

    ntok = w.batch * w.seq_len
    tps = ntok / (ms_per_step / 1e3)
    mflop = model_flops_per_token(w)
    frac = tps * mflop / PEAK_BF16_FLOPS

    roof = None
    if kern_n > 0 and roof_k.get("bound", "mfma") == "hbm":
        nbytes = roof_k["bytes"](w) * steps_timed
        achieved = nbytes / (kern_ms / 1e3) / 1e9
        roof = {"kernel": roof_k["desc"], "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                "frac": round(achieved / (PEAK_HBM_BYTES / 1e9), 4),
                "traffic": None, "launches": kern_n,
                "timed_over": f"{steps_timed} eager steps " + ("after the timed region" if graph
                                                                else "of the timed region"),
                "avg_launch_ms": round(kern_ms / kern_n, 4),
                "algorithmic_bytes_per_launch": round(nbytes / kern_n)}
    elif kern_n > 0:
        flops = roof_k["flops"](w) * steps_timed
        achieved = flops / (kern_ms / 1e3) / 1e12
        traffic = None
        if roof_k["pmc"] and w.name == "d12" and not (w.smear or w.backout):
            from decoder_only_pretraining_amd.profiling import traffic_for
            traffic = traffic_for(os.path.join(ROOT, roof_k["pmc"]))
        peak = PEAK_FP8_FLOPS if (roof_k.get("fp8_peak") and w.fp8_linears) else PEAK_BF16_FLOPS
        roof = {"kernel": roof_k["desc"] + (" in fp8 (e4m3 / e5m2 MFMA)" if peak == PEAK_FP8_FLOPS
                                            else ""),
                "bound": "mfma", "achieved": round(achieved, 1),
                "peak": peak / 1e12, "unit": "TFLOP/s",
                "frac": round(achieved / (peak / 1e12), 4),
                "traffic": traffic, "launches": kern_n,
                "timed_over": f"{steps_timed} eager steps " + ("after the timed region" if graph
                                                                else "of the timed region"),
                "avg_launch_ms": round(kern_ms / kern_n, 4),
                "algorithmic_flop_per_launch": round(flops / kern_n)}

    metric = METRIC if w.name == "d12" else METRIC.replace("d12", w.name)
    out = {
        "metric": metric, "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "ms_per_step_median": round(float(np.median(per_step)), 3),
        "ms_per_step_p10": round(float(np.percentile(per_step, 10)), 3),
        "ms_per_step_p90": round(float(np.percentile(per_step, 90)), 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 linears (e4m3/e5m2), bf16 elsewhere" if w.fp8_linears else "bf16",
        "data": "synthetic (seeded Zipf(1.1) tokens, N(0,0.02) weights)",
        "config": {"workload": f"{w.name}: {w.n_layer} layers, n_embd {w.n_embd}, heads "
                               f"{w.n_head}/{w.n_kv_head}, head_dim {w.head_dim}, MLP "
                               f"{w.mlp_hidden}, vocab {w.vocab}, seq {w.seq_len}, batch "
                               f"{w.batch}, window {w.short_window}"
                               + (", fp8 block linears" if w.fp8_linears else "")
                               + (", smear" if w.smear else "")
                               + (", backout (lambda 0.5)" if w.backout else ""),
                   "seq_len": w.seq_len, "batch": w.batch, "tokens_per_step": ntok,
                   "parallelism": "none (1 GPU)"},
        "launch": "HIP graph replay of the call (GPT_F_GRAPH)" if graph else "eager",
        "mfma_util_vs_bf16_peak": round(frac, 4),
        "model_mflop_per_token": round(mflop / 1e6, 3),
        "loss": round(loss, 5),
        "roofline": roof,
        "context": {"pages_rtx4070_full_step_tokens_per_s": 55670},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, params, tokens, targets, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
