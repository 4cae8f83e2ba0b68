#!/usr/bin/env python3
"""Prefill throughput of the Llama-3-8B-shaped decoder on one MI355X.

One step = one fwd_prefill of the whole forward pass over a batch of 8 x 2048
synthetic token ids (32 layers, hidden 4096, 32/8 heads, head_dim 128, FFN 14336,
vocab 128256, bf16 weights N(0, 0.02)), writing fp32 logits, per-position argmax
and the fp32 hidden slots. Inputs are resident in HBM before the timed region.

Prints ONE JSON line with tokens/s, the roofline record of the dominant kernel
(gate/up projection + SwiGLU, timed with HIP events on the library's stream) and
the CPU oracle's throughput on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix (and vector) peak
PEAK_HBM_GBS = 8000.0
METRIC = "prefill tokens/s (Llama-3-8B shape, bf16); GEMM MFMA util vs peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_flops(cfg, B, S):
    """Algorithmic flops of each kernel class for one prefill (multiply-add = 2)."""
    T = B * S
    H, Hq, Hkv, D, F, V, L = cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab, cfg.n_layers
    kinds = cfg.kinds()
    attn = 0
    for l in range(L):
        W = cfg.sliding_window if kinds[l] == "local" else 0
        visible = sum(min(i + 1, W) if W > 0 else i + 1 for i in range(S))
        attn += 4 * D * Hq * B * visible
    return {
        "qkv_rope": L * 2 * T * H * (Hq + 2 * Hkv) * D,
        "attention": attn,
        "o_proj": L * 2 * T * Hq * D * H,
        "gate_up": L * 2 * T * H * 2 * F,
        "down_proj": L * 2 * T * F * H,
        "lm_head": 2 * T * H * V,
    }


def cpu_baseline(cfg, S):
    """The CPU oracle (as it stands) on a bounded sample: one S-token row through
    the embedding, final norm and LM head with 0 layers, then with 1 layer; the
    difference prices one layer. Full-model seconds per row = t0 + L * t_layer."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from synth import workloads as wl

    ids = wl.draw_ids(cfg)[:1, :S]
    times = {}
    for n in (0, 1):
        c = cfg.replace(n_layers=n)
        w = wl.LazyWeights(c, cache=True)
        for name in wl.weight_shapes(c):
            w[name]                                   # draw outside the timed region
        t = time.perf_counter()
        oracle.forward(c, w, ids, want_logits=True, want_hidden=False)  # head included
        times[n] = time.perf_counter() - t
        del w
    t_layer = max(times[1] - times[0], 1e-9)
    per_row = times[0] + cfg.n_layers * t_layer
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    nproc, model = cpu_info()
    return {
        "value": S / per_row,
        "unit": "tokens/s",
        "cores": threads,
        "nproc": nproc,
        "cpu_model": model,
        "kind": "oracle",
        "sample": (f"1 row x {S} tokens: embedding+final norm+LM head ({times[0]:.1f} s) and one decoder layer "
                   f"({t_layer:.1f} s) timed, scaled to {cfg.n_layers} layers; float64 numpy oracle"),
    }


def decode_leg(fwd, model, cfg, ids, steps, stream):
    """Greedy decode on a cached session: prefill the batch's prompts, then `steps`
    one-token steps for every row, each fed the previous step's argmax (host ids, as
    the API takes them). Every step reads all weights and the whole cache: HBM-bound."""
    import torch
    B, S = ids.shape
    with torch.cuda.stream(stream):
        sess = fwd.Session(model, max_batch=B, max_seq=S + steps + 2)
        first = sess.prefill(ids, logits=False, argmax=True)
        tok = first["argmax"][:, -1].cpu().numpy()
        tok = sess.decode(tok, logits=False, argmax=True)["argmax"][:, 0].cpu().numpy()   # warm-up step
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            tok = sess.decode(tok, logits=True, argmax=True)["argmax"][:, 0].cpu().numpy()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t
        sess.close()
    sizes = fwd.output_sizes(cfg, B, S)
    ctx = S + 1 + steps / 2.0                      # mean cached length over the timed steps
    kv = 2 * cfg.n_layers * B * cfg.n_kv_heads * ctx * cfg.head_dim * 2
    per_step = sizes["weight_bytes"] + kv
    ms = elapsed * 1000.0 / steps
    log(f"decode: {steps} steps of {B} tokens at context {S}: {ms:.2f} ms/step")
    return {"tokens_per_s": B * steps / elapsed, "ms_per_step": ms, "batch": B, "context": S, "steps": steps,
            "bound": "hbm", "bytes_per_step": per_step, "achieved_gbs": per_step / (ms * 1e-3) / 1e9,
            "peak_gbs": PEAK_HBM_GBS, "frac": per_step / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "note": "bytes = all packed weights + the cached keys and values read once per step"}


def variant_leg(fwd, cfg0, ids, steps, stream):
    """The Llama-3-8B shape with the family variants switched on (QK-norm, tanh-GELU
    gating, llama3 frequency bands at original context 8192, factor 8): tokens/s of the
    same prefill, and the QK-norm pass against HBM (it reads and writes every q and k
    head once: T * (Hq + Hkv) * D * 2 B each way per layer)."""
    import torch
    from synth import workloads as wl
    cfg = cfg0.replace(qk_norm=True, ffn_act="gelu_tanh", rope_scaling="llama3", rope_factor=8.0,
                       rope_low_freq_factor=1.0, rope_high_freq_factor=4.0, rope_original_max_pos=8192,
                       name="llama3-8b-shape-variants")
    B, S = ids.shape
    T = B * S
    weights = {n: fwd.to_device(wl.draw_weight(cfg, n)) for n in wl.weight_shapes(cfg)}
    model = fwd.Model(cfg, weights, max_tokens=T, stream=stream)
    del weights
    torch.cuda.empty_cache()
    argmax = torch.empty((B, S), dtype=torch.int32, device="cuda")
    model.prefill_into(ids, None, None, argmax)                       # warm-up
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        model.prefill_into(ids, None, None, argmax)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1000.0 / steps
    model.set_timing(True)
    model.prefill_into(ids, None, None, argmax)
    torch.cuda.synchronize()
    timing = model.timing()
    model.set_timing(False)
    model.close()
    qk = timing["qk_norm"]
    qk_bytes = 2 * T * (cfg.n_heads + cfg.n_kv_heads) * cfg.head_dim * 2
    qk_us = qk["ms"] * 1000.0 / max(qk["launches"], 1)
    log(f"variants: {ms:.2f} ms/step, QK-norm pass {qk_us:.1f} us per layer")
    return {"config": "llama3-8b-shape prefill 8 x 2048 with QK-norm, tanh-GELU gating, llama3 rope scaling "
                      "(factor 8, original context 8192); argmax only",
            "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms,
            "kernels_ms_per_step": {k: v["ms"] for k, v in timing.items() if v["launches"]},
            "qk_norm_pass": {"us_per_layer": qk_us, "bytes_per_layer": qk_bytes, "bound": "hbm",
                             "achieved_gbs": qk_bytes / (qk_us * 1e-6) / 1e9, "peak_gbs": PEAK_HBM_GBS,
                             "frac": qk_bytes / (qk_us * 1e-6) / 1e9 / PEAK_HBM_GBS}}


def moe_leg(fwd, steps, stream):
    """Mixture-of-experts layers at a 30B-A3B-style shape (hidden 2048, 32/4 heads x 128,
    128 experts of width 768, top-8, vocab 151936), a 4-layer slice, prefill 8 x 2048:
    per-kernel-class times and the grouped expert products against the bf16 peak
    (algorithmic flops: 2 * T * k * H * 2 F_e for gate/up plus 2 * T * k * F_e * H for
    down per layer)."""
    import torch
    from synth import workloads as wl
    cfg = wl.ModelConfig("moe-30b-a3b-shape-4L", 4, 2048, 32, 4, 128, 6144, 151936, rope_theta=1e6, qk_norm=True,
                         n_experts=128, n_experts_per_tok=8, moe_ffn=768, batch=8, seq=2048)
    B, S = cfg.batch, cfg.seq
    T = B * S
    weights = {n: fwd.to_device(wl.draw_weight(cfg, n)) for n in wl.weight_shapes(cfg)}
    model = fwd.Model(cfg, weights, max_tokens=T, stream=stream)
    del weights
    torch.cuda.empty_cache()
    ids = wl.draw_ids(cfg)
    argmax = torch.empty((B, S), dtype=torch.int32, device="cuda")
    model.prefill_into(ids, None, None, argmax)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        model.prefill_into(ids, None, None, argmax)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1000.0 / steps
    model.set_timing(True)
    model.prefill_into(ids, None, None, argmax)
    torch.cuda.synchronize()
    timing = model.timing()
    model.set_timing(False)
    model.close()
    k, H, Fe, L = cfg.n_experts_per_tok, cfg.hidden, cfg.moe_ffn, cfg.n_layers
    expert_flops = L * (2 * T * k * H * 2 * Fe + 2 * T * k * Fe * H)
    ex = timing["moe_experts"]["ms"]
    log(f"moe: {ms:.2f} ms per 4-layer step, expert products {ex:.2f} ms")
    return {"config": "4 layers of a MoE shape: hidden 2048, 32/4 heads x 128 (QK-norm), 128 experts x 768, top-8, "
                      "vocab 151936; prefill 8 x 2048, argmax only",
            "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "kernels_ms_per_step": {n: v["ms"] for n, v in timing.items() if v["launches"]},
            "expert_products": {"bound": "mfma", "tflops": expert_flops / (ex * 1e-3) / 1e12,
                                "frac": expert_flops / (ex * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                "algorithmic_tflop_per_step": expert_flops / 1e12}}


def gemm_sweep_leg(fwd, stream, calls):
    """The standalone projection Y = X·Wᵀ over the [P, in, out] sweep (bf16 N(0, 1)
    operands, fp32 output): per shape, after ~0.2 s of warm-up calls, the median of
    `calls` fwd_gemm launches, each bracketed by HIP events on the stream the call runs
    on; TFLOP/s by algorithmic flops
    2 P in out, against the bf16 peak, and the achieved HBM rate by algorithmic bytes
    2 (P in + out in) + 4 P out."""
    import torch
    from synth import workloads as wl
    out = []
    for P, K, N in wl.GEMM_SWEEP:
        Xh, Wh = wl.draw_gemm(P, K, N)
        X, W = fwd.to_device(Xh), fwd.to_device(Wh)
        del Xh, Wh
        Y = torch.empty((P, N), dtype=torch.float32, device="cuda")
        with torch.cuda.stream(stream):
            # the GPU idles while the operands are drawn on the host: warm up for ~0.2 s of
            # calls (at least 3), so that the timed calls run at the steady-state clock
            t0, n = time.perf_counter(), 0
            while n < 3 or (time.perf_counter() - t0 < 0.2 and n < 5000):
                for _ in range(8):
                    fwd.gemm(X, W, Y, stream=stream)
                n += 8
                stream.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
            for a, b in ev:
                a.record(stream)
                fwd.gemm(X, W, Y, stream=stream)
                b.record(stream)
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)
        med = ms[len(ms) // 2]
        flops, nbytes = 2.0 * P * K * N, 2.0 * (P * K + N * K) + 4.0 * P * N
        tf = flops / (med * 1e-3) / 1e12
        out.append({"shape_P_in_out": [P, K, N], "calls": calls, "median_us": med * 1e3, "min_us": ms[0] * 1e3,
                    "tflops": tf, "frac_of_bf16_peak": tf / PEAK_BF16_TFLOPS,
                    "achieved_gbs": nbytes / (med * 1e-3) / 1e9})
        log(f"gemm [{P},{K},{N}]: {med * 1e3:.1f} us median of {calls}, {tf:.1f} TFLOP/s "
            f"({tf / PEAK_BF16_TFLOPS:.3f} of peak)")
        del X, W, Y
        torch.cuda.empty_cache()
    return out


def cpu_info():
    """(logical CPUs, CPU model name) of this host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_oracle_other_workloads():
    """The oracle on the other workloads, each bounded to seconds: the tiny fp32 model
    and the SmolLM2-shaped model in full, the Gemma3-style model as embedding + final
    norm + head and one layer scaled to 48 layers (as the Llama sample), and the GEMM
    sweep (the two large shapes on 256 rows of X, scaled to P rows: every output row is
    an independent product)."""
    import numpy as np

    import oracle
    from synth import bf16_bits_to_f32
    from synth import workloads as wl
    res = {}
    for cfg in (wl.TINY_F32, wl.SMOLLM2_135M):
        w = wl.LazyWeights(cfg, cache=True)
        for name in wl.weight_shapes(cfg):
            w[name]
        ids = wl.draw_ids(cfg)
        t = time.perf_counter()
        oracle.forward(cfg, w, ids, want_hidden=False)
        dt = time.perf_counter() - t
        res[cfg.name] = {"tokens_per_s": ids.size / dt, "seconds": dt, "sample": f"full prefill {ids.shape}"}
        del w
    cfg = wl.GEMMA3_STYLE
    ids = wl.draw_ids(cfg)
    times = {}
    for n in (0, 1):
        c = cfg.replace(n_layers=n, layer_kind=cfg.layer_kind[:n])
        w = wl.LazyWeights(c, cache=True)
        for name in wl.weight_shapes(c):
            w[name]
        t = time.perf_counter()
        oracle.forward(c, w, ids, want_hidden=False)
        times[n] = time.perf_counter() - t
        del w
    per = times[0] + cfg.n_layers * max(times[1] - times[0], 1e-9)
    res[cfg.name] = {"tokens_per_s": ids.size / per, "seconds_extrapolated": per,
                     "sample": f"1 x {ids.shape[1]} tokens: head ({times[0]:.1f} s) + one layer, scaled to 48 layers"}
    sweep = []
    for P, K, N in wl.GEMM_SWEEP:
        Xh, Wh = wl.draw_gemm(P, K, N)
        rows = min(P, 256)
        X, W = bf16_bits_to_f32(Xh[:rows]), bf16_bits_to_f32(Wh)
        t = time.perf_counter()
        oracle.gemm(X, W)
        dt = (time.perf_counter() - t) * P / rows
        sweep.append({"shape_P_in_out": [P, K, N], "seconds": dt, "gflops": 2.0 * P * K * N / dt / 1e9,
                      "sample": f"{rows} of {P} rows" + (", scaled" if rows < P else "")})
        del X, W, Xh, Wh
    res["gemm_sweep"] = sweep
    return res


def forward_flops(cfg, B, S):
    """Algorithmic flops of one prefill: the projections, the head and the attention
    contractions over the visible (causal, windowed) key pairs."""
    return sum(kernel_flops(cfg, B, S).values())


def configs_leg(fwd, steps, stream):
    """The other forward configurations at their own shapes: the tiny fp32 model (2
    layers, 1 x 16), the SmolLM2-shaped model (30 layers, 1 x 512) and the Gemma3-style
    model (48 layers, 5 local : 1 global, sandwich norms, softcap 30, 1 x 1024): ms per
    prefill (argmax only), tokens/s and the fraction of the peak of the computing
    dtype (fp32 matrix for the tiny model, bf16 otherwise) by algorithmic flops."""
    import torch
    from synth import workloads as wl
    out = {}
    for cfg in (wl.TINY_F32, wl.SMOLLM2_135M, wl.GEMMA3_STYLE):
        B, S = cfg.batch, cfg.seq
        ids = wl.draw_ids(cfg)
        weights = {n: fwd.to_device(wl.draw_weight(cfg, n)) for n in wl.weight_shapes(cfg)}
        model = fwd.Model(cfg, weights, max_tokens=B * S, stream=stream)
        del weights
        torch.cuda.empty_cache()
        argmax = torch.empty((B, S), dtype=torch.int32, device="cuda")
        for _ in range(2):
            model.prefill_into(ids, None, None, argmax)                   # warm-up
        torch.cuda.synchronize()
        n = max(steps, 1) * (10 if S * B <= 512 else 2)
        t = time.perf_counter()
        for _ in range(n):
            model.prefill_into(ids, None, None, argmax)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t) * 1000.0 / n
        model.close()
        del argmax
        torch.cuda.empty_cache()
        fl = forward_flops(cfg, B, S)
        log(f"{cfg.name}: {ms:.3f} ms per prefill of {B} x {S}")
        rec = {"batch": B, "seq": S, "ms_per_step": ms, "tokens_per_s": B * S / (ms * 1e-3),
               "algorithmic_tflop_per_step": fl / 1e12, "tflops": fl / (ms * 1e-3) / 1e12,
               "outputs": "argmax only"}
        if cfg.dtype == "f32":
            rec["frac_of_f32_peak"] = rec["tflops"] / PEAK_F32_TFLOPS
        else:
            rec["frac_of_bf16_peak"] = rec["tflops"] / PEAK_BF16_TFLOPS
        out[cfg.name] = rec
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hidden", action="store_true", help="skip the hidden-slot output")
    ap.add_argument("--timing-steps", type=int, default=2, help="extra steps timed per kernel with HIP events")
    ap.add_argument("--decode-steps", type=int, default=16,
                    help="greedy decode steps timed on a cached session after the prefill (0: skip)")
    ap.add_argument("--variant-leg", action="store_true",
                    help="also time the same shape with QK-norm, tanh-GELU gating and llama3 rope scaling")
    ap.add_argument("--moe-leg", action="store_true", help="also time mixture-of-experts layers (4-layer slice)")
    ap.add_argument("--configs-leg", action="store_true",
                    help="also time the SmolLM2-shaped (1 x 512) and Gemma3-style (1 x 1024) prefills")
    ap.add_argument("--gemm-calls", type=int, default=20,
                    help="fwd_gemm calls timed per shape of the standalone GEMM sweep (0: skip the sweep)")
    args = ap.parse_args()
    if args.timing_steps < 1:
        ap.error("--timing-steps must be at least 1 (the roofline comes from those steps)")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the batch rows are independent: more GPUs would each run their own share)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from decoder_only_transformer_bf16_amd import fwd
    from synth import workloads as wl

    cfg = wl.LLAMA3_8B
    B, S = cfg.batch, cfg.seq
    T = B * S
    torch.cuda.set_device(0)
    if not fwd.available():
        raise SystemExit("libfwd.so sees no gfx950 device")

    t0 = time.time()
    weights = {}
    for name in wl.weight_shapes(cfg):
        weights[name] = fwd.to_device(wl.draw_weight(cfg, name))
    stream = torch.cuda.Stream()
    model = fwd.Model(cfg, weights, max_tokens=T, stream=stream)
    del weights
    torch.cuda.empty_cache()
    ids = wl.draw_ids(cfg)
    logits = torch.empty((B, S, cfg.vocab), dtype=torch.float32, device="cuda")
    argmax = torch.empty((B, S), dtype=torch.int32, device="cuda")
    hidden = None if args.no_hidden else torch.empty((cfg.n_layers + 2, B, S, cfg.hidden), dtype=torch.float32,
                                                     device="cuda")
    log(f"setup {time.time() - t0:.1f} s (weights drawn, uploaded, packed)")

    for i in range(args.warmup):
        model.prefill_into(ids, logits, hidden, argmax)
        log(f"warmup {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(args.steps):
        model.prefill_into(ids, logits, hidden, argmax)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t
    ms_per_step = elapsed * 1000.0 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.2f} ms/step")
    # the same prefill returning only the per-position argmax (no logits, no slots)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(args.steps):
        model.prefill_into(ids, None, None, argmax)
    torch.cuda.synchronize()
    ms_argmax_only = (time.perf_counter() - t) * 1000.0 / args.steps
    log(f"argmax-only outputs: {ms_argmax_only:.2f} ms/step")
    # per-kernel breakdown from separate steps with HIP events around every launch
    # (the events add gaps, so these steps are not part of the throughput figure)
    model.set_timing(True)
    for i in range(args.timing_steps):
        model.prefill_into(ids, logits, hidden, argmax)
    torch.cuda.synchronize()
    timing = model.timing()
    model.set_timing(False)

    flops = kernel_flops(cfg, B, S)
    total_flops = sum(flops.values())
    kernels = {}
    for k, v in timing.items():
        if not v["launches"]:
            continue
        rec = {"ms_per_launch": v["ms"] / v["launches"], "launches_per_step": v["launches"] / args.timing_steps,
               "ms_per_step": v["ms"] / args.timing_steps}
        if k in flops:
            per_launch = flops[k] / (v["launches"] / args.timing_steps)
            rec["tflops"] = per_launch / (rec["ms_per_launch"] * 1e-3) / 1e12
            rec["frac_of_bf16_peak"] = rec["tflops"] / PEAK_BF16_TFLOPS
        kernels[k] = rec
    dom = kernels["gate_up"]
    gate_up_flops_per_launch = 2 * T * cfg.hidden * 2 * cfg.ffn
    achieved = gate_up_flops_per_launch / (dom["ms_per_launch"] * 1e-3) / 1e12

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "gate_up_swiglu_llama3_8b_traffic.json")
    if os.path.exists(tfile):
        try:
            tr = json.load(open(tfile))
            from decoder_only_transformer_bf16_amd import _build
            if tr.get("source_digest") == _build.source_digest():
                traffic = tr["bytes_per_launch"]
        except Exception as e:  # stale or unreadable record: report none
            log(f"traffic record ignored: {e}")

    result = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, uniform token ids)",
        "config": {"workload": "llama3-8b-shape prefill: 8 x 2048 tokens, 32 layers, hidden 4096, 32/8 heads x 128, "
                               "ffn 14336, vocab 128256; outputs fp32 logits, argmax"
                               + ("" if args.no_hidden else ", fp32 hidden slots"),
                   "batch": B, "seq_len": S, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "gate_up projection + SwiGLU epilogue [16384, 4096 -> 2 x 14336]",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic},
        "end_to_end": {"algorithmic_tflop_per_step": total_flops / 1e12,
                       "tflops": total_flops / (ms_per_step * 1e-3) / 1e12,
                       "frac_of_bf16_peak": total_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "kernels": kernels,
        "modes": {"all_outputs": {"ms_per_step": ms_per_step, "tokens_per_s": T * args.steps / elapsed,
                                  "outputs": "fp32 logits, argmax" + ("" if args.no_hidden else ", hidden slots")},
                  "argmax_only": {"ms_per_step": ms_argmax_only, "tokens_per_s": T / (ms_argmax_only * 1e-3),
                                  "outputs": "argmax only (folded into the LM-head epilogue; no logits or slots written)"}},
    }
    if args.decode_steps > 0:
        del logits, hidden
        torch.cuda.empty_cache()
        result["decode"] = decode_leg(fwd, model, cfg, ids, args.decode_steps, stream)
    model.close()
    del argmax
    torch.cuda.empty_cache()
    if args.variant_leg:
        result["variants"] = variant_leg(fwd, cfg, ids, max(args.steps, 1), stream)
        torch.cuda.empty_cache()
    if args.moe_leg:
        result["moe"] = moe_leg(fwd, max(args.steps, 1), stream)
        torch.cuda.empty_cache()
    if args.configs_leg:
        result["configs"] = configs_leg(fwd, max(args.steps, 1), stream)
        torch.cuda.empty_cache()
    if args.gemm_calls > 0:
        result["gemm_sweep"] = gemm_sweep_leg(fwd, stream, max(args.gemm_calls, 20))
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(cfg, S)
        log("cpu oracle on the other workloads (bounded samples)")
        result["cpu_baseline"]["other_workloads"] = cpu_oracle_other_workloads()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
