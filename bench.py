"""Throughput of the Qwen2 decoder forward on one MI355X.

A step is one pass of the whole hot path over one batch: prefill of the
batch's prompts (the TTFT token), then the workload's greedy decode steps,
each through the C ABI of libqw.so.  Inputs (weights, token ids) are seeded
synthetic data resident in HBM before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1.5b-longctx]

The default workload is the largest one that fits one GPU: Qwen2.5-1.5B
shapes, batch 32 x 8192 prompt tokens, 128 greedy decode steps.

Prints one JSON line.  `value` is decode tokens/s over the timed steps;
prefill tokens/s and TTFT ride along.  `roofline` covers the kernel family
with the most decode time, timed with HIP events on the model's stream over
an extra, eagerly launched pass (same kernels, same data); the whole decode
step and the prefill's dominant GEMM get roofline objects of their own.
Fractions are given against the published peaks and against peaks measured
in the same run (an HBM copy and an MFMA-only loop).  `cpu_baseline` is the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic as S  # noqa: E402

METRIC = "decode tokens/s + prefill tokens/s (TTFT) at 1 MI355X; % HBM / MFMA roofline"
HBM_PEAK_GBS = 8000.0
# committed rocprofv3 counter summaries (FETCH_SIZE / WRITE_SIZE per launch)
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "*_hbm_traffic.json")
MFMA_F16_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "1.5b-longctx"
DESCRIPTIONS = {
    "tiny": "tiny Qwen2-style decoder, fp32 (2 layers, hidden 128), batch 1, prompt 16, 8 greedy decode steps",
    "0.5b": "Qwen2.5-0.5B shapes, bf16 weights, batch 1, prompt 128, 128 greedy decode steps, cache 2048",
    "1.5b": "Qwen2.5-1.5B shapes, bf16 weights, batch 1, prompt 512, 256 greedy decode steps, cache 1024",
    "1.5b-prefill": "Qwen2.5-1.5B shapes, bf16 weights, batch 8 x prompt 2048, 32 greedy decode steps, cache 4096",
    "1.5b-longctx": "Qwen2.5-1.5B shapes, bf16 weights, batch 32 x prompt 8192, 128 greedy decode steps, cache 8320",
    "coder-7b": "Qwen2.5-Coder-7B shapes (untied LM head), bf16 weights, batch 1, prompt 512, 128 greedy decode "
                "steps, cache 1024",
}


def decode_family_bytes(w: S.Workload, family: str, ctx_mean: float) -> float:
    """Algorithmic HBM bytes of ONE launch of a decode kernel family: every
    weight element once (its storage size), the B activation rows in and out,
    and for attention the K and V rows of the live context."""
    m, B = w.model, w.batch
    e = 2 if m.dtype == "bf16" else 4
    H, I, V, qd, kvd = m.hidden, m.intermediate, m.vocab, m.q_dim, m.kv_dim
    nqkv = qd + 2 * kvd
    if family == "gemm_qkv":
        return nqkv * H * e + B * H * e + B * nqkv * 4
    if family == "gemm_o":
        return H * qd * e + B * qd * e + 2 * B * H * 4
    if family == "gemm_gate_up":
        return 2 * I * H * e + B * H * e + B * I * e
    if family == "gemm_down":
        return H * I * e + B * I * e + 2 * B * H * 4
    if family == "attn_o":   # attention + o projection in one launch (1-2 rows, short context)
        return (B * m.n_kv_heads * ctx_mean * m.head_dim * e * 2 + H * qd * e + B * nqkv * 8
                + 2 * B * H * 8)
    if family == "mlp":   # norm + gate/up + SwiGLU + down in one launch (1-2 rows)
        return 3 * I * H * e + B * H * 8 * 2
    if family == "lm_head":
        return V * H * e + B * H * e + B * V * 4
    if family == "attention":
        return B * m.n_kv_heads * ctx_mean * m.head_dim * e * 2 + 2 * B * qd * e
    return float("nan")


def measured_traffic(workload: str, family: str, pattern: str = None):
    """HBM bytes per launch of a kernel family from a committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads
    for a copy of known size), or None when no summary covers this workload
    and family, or the kernel's source file has changed since it was taken."""
    for path in sorted(glob.glob(pattern or TRAFFIC_GLOB)):
        try:
            with open(path) as f:
                d = json.load(f)
            if d.get("workload") != workload or d.get("family") != family:
                continue
            with open(os.path.join(ROOT, d["kernel_source"]), "rb") as f:
                sha = hashlib.sha256(f.read()).hexdigest()
        except (OSError, ValueError, KeyError):
            continue
        if sha == d.get("kernel_source_sha256"):
            return int(d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"])
    return None


def decode_step_bytes(w: S.Workload, ctx_mean: float) -> float:
    """Algorithmic HBM bytes of one whole decode step: every weight once (all
    layers and the LM head), the live K/V context of every sequence read, and
    the new K/V rows written."""
    m, B = w.model, w.batch
    e = 2 if m.dtype == "bf16" else 4
    H, I, V, qd, kvd = m.hidden, m.intermediate, m.vocab, m.q_dim, m.kv_dim
    per_layer = H * (qd + 2 * kvd) + qd * H + 3 * H * I
    weights = e * (m.n_layers * per_layer + V * H)
    kv = B * m.n_layers * 2 * kvd * e * (ctx_mean + 1)
    return weights + kv


def prefill_family_flops(w: S.Workload, family: str) -> float:
    """Algorithmic FLOP of ONE prefill launch of a kernel family (T = B*P
    rows): 2*M*N*K for the projections, causal QK^T + PV for attention."""
    m, B, P = w.model, w.batch, w.prompt_len
    T = B * P
    H, I, V, qd, kvd = m.hidden, m.intermediate, m.vocab, m.q_dim, m.kv_dim
    if family == "gemm_qkv":
        return 2.0 * T * (qd + 2 * kvd) * H
    if family == "gemm_o":
        return 2.0 * T * H * qd
    if family == "gemm_gate_up":
        return 2.0 * T * 2 * I * H
    if family == "gemm_down":
        return 2.0 * T * H * I
    if family == "lm_head":
        return 2.0 * B * V * H
    if family == "attention":
        return 2.0 * B * m.n_heads * m.head_dim * P * (P + 1)
    return float("nan")


def run_step(model, ids, toks, D, torch, ev=None):
    """prefill + D decode steps; ev = (start, after_prefill, end) events."""
    if ev:
        ev[0].record()
    model.prefill(ids, next_ids=toks[0])
    if ev:
        ev[1].record()
    for s in range(D):
        model.decode_step(toks[s], next_ids=toks[s + 1])
    if ev:
        ev[2].record()


def cpu_info():
    """CPU model name and the number of cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


# Prompt tokens of the oracle's sample: its decode rate is set by streaming
# every weight once per token (12.3 GB in float64 at 1.5B shapes), which a
# context of this size already shows; an 8k-token float64 prefill alone takes
# minutes.
CPU_SAMPLE_PROMPT = 512


def cpu_baseline(w: S.Workload, W, ids, budget_s: float = 15.0):
    """The oracle, untuned, on a bounded sample of batch row 0: prefill of
    its first CPU_SAMPLE_PROMPT prompt tokens, then decode steps until the
    time budget is spent.  Reports decode tokens/s of the sample."""
    import oracle as O
    from threadpoolctl import threadpool_info
    blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model_name, affinity = cpu_info()
    P = min(w.prompt_len, CPU_SAMPLE_PROMPT)
    om = O.OracleModel(w.model, W)
    cache = om.new_cache(P + w.decode_steps)
    t0 = time.perf_counter()
    lg = om.forward(ids[0, :P], 0, cache)
    t_prefill = time.perf_counter() - t0
    tok = O.greedy_token(lg)
    n, t1 = 0, time.perf_counter()
    while n < w.decode_steps and (time.perf_counter() - t1) < budget_s:
        lg = om.forward([tok], P + n, cache)
        tok = O.greedy_token(lg)
        n += 1
    t_dec = time.perf_counter() - t1
    # the oracle's attention runs one thread per head (at most the affinity
    # count); its matrix products use the BLAS pool
    cores = max(blas_threads, min(w.model.n_heads, affinity))
    return {"value": round(n / t_dec, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": model_name, "sched_affinity_cores": affinity, "blas_threads": blas_threads,
            "sample": f"batch row 0 of {w.batch}: the first {P} of its {w.prompt_len} prompt tokens prefilled "
                      f"({P / t_prefill:.1f} tokens/s, {t_prefill * 1e3:.0f} ms), then the first {n} greedy "
                      f"decode steps (float64 numpy oracle; decode tokens/s)"}


def measure_peaks(torch, Q):
    """HBM copy rate (GB/s) and MFMA-only fp16 rate (TFLOP/s) measured now,
    on this GPU, by the library's peak helpers."""
    n = 1 << 30
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream().cuda_stream
    Q.qw_peak_copy(dst.data_ptr(), src.data_ptr(), n, 2, False, st)      # warm
    copy = Q.qw_peak_copy(dst.data_ptr(), src.data_ptr(), n, 10, False, st)
    read = Q.qw_peak_copy(dst.data_ptr(), src.data_ptr(), n, 10, True, st)
    del src, dst
    Q.qw_peak_mfma(2000, st)
    tflops = Q.qw_peak_mfma(100000, st)
    return {"read_GBps": round(read, 1), "copy_GBps": round(copy, 1), "bytes": n,
            "mfma_f16_TFLOPs": round(tflops, 1),
            "mfma": "8192 waves x 100000 rounds of 8 independent v_mfma_f32_16x16x32_f16"}


def cache_compare(torch, Q, w: S.Workload, steps: int, reps: int, warmup: int):
    """Greedy generation of `steps` tokens after the workload's prompts, with
    the KV cache (one prefill, then decode steps) and without it (a prefill
    over the whole sequence at every step), each timed over `reps` runs with
    HIP events: the pages' cache benchmark ("augur", cache benchmarking:
    generation speed, prefill and decode time, cached against uncached)."""
    m = w.model
    B, P = w.batch, w.prompt_len
    W = S.make_weights(m, w.weight_seed)
    model = Q.Model(m, Q.device_tensors(m, W), B, P + steps + 1)
    ids = torch.from_numpy(S.make_ids(w)).cuda()
    out = {}
    toks = {}
    for use_cache in (True, False):
        for _ in range(warmup):
            model.generate(ids, steps, use_cache=use_cache)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            t = model.generate(ids, steps, use_cache=use_cache)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        key = "cached" if use_cache else "uncached"
        toks[key] = t.cpu().numpy()
        out[key] = {"ms_per_generation": round(ms, 3), "new_tokens_per_s": round(B * (steps + 1) / (ms / 1e3), 1)}
    model.close()
    agree = (toks["cached"] == toks["uncached"]).all(axis=1)
    return {"metric": "greedy generation with and without the KV cache", "workload": w.name, "batch": B,
            "prompt_len": P, "new_tokens": steps + 1, "reps": reps, **out,
            "speedup": round(out["uncached"]["ms_per_generation"] / out["cached"]["ms_per_generation"], 2),
            "rows_with_identical_tokens": int(agree.sum())}


def ragged_compare(torch, Q, name: str, reps: int, warmup: int, padded: bool = True):
    """A ragged batch (prompts of different lengths, packed, no padding) on
    the paged KV cache, against the same prompts padded to the longest one on
    the dense cache (what a batch without ragged support computes): prefill
    time, decode step time, and the cache each needs.  Useful tokens only
    count toward the rates of both."""
    rw = S.RAGGED_WORKLOADS[name]
    m, n, D = rw.model, rw.n, rw.decode_steps
    lens, prompts = rw.lengths(), rw.prompts()
    L_max, T = max(lens), sum(lens)
    max_seq = L_max + D
    W = S.make_weights(m, rw.weight_seed)
    tensors = Q.device_tensors(m, W)
    blk = Q.QW_KV_BLOCK
    n_blocks = sum((x + D + blk - 1) // blk for x in lens)
    kv_elem_bytes = 2 * m.n_layers * m.kv_dim * 2        # K and V, all layers, f16, per position

    def timed_runs(model, prefill):
        toks = torch.empty((D + 1, n), dtype=torch.int32, device="cuda")

        def one(ev=None):
            if ev:
                ev[0].record()
            prefill(toks[0])
            if ev:
                ev[1].record()
            for k in range(D):
                model.decode_step(toks[k], next_ids=toks[k + 1])
            if ev:
                ev[2].record()
        for _ in range(warmup):
            one()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        for e in evs:
            one(e)
        torch.cuda.synchronize()
        return (float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
                float(np.mean([e[1].elapsed_time(e[2]) for e in evs])))

    print(f"[bench] ragged {name}: {n} prompts, {T} tokens (longest {L_max}), paged cache", file=sys.stderr,
          flush=True)
    model = Q.Model(m, tensors, n, max_seq, kv_blocks=n_blocks)
    ids = torch.from_numpy(np.concatenate(prompts)).cuda()
    r_pre, r_dec = timed_runs(model, lambda out: model.prefill_ragged(ids, lens, next_ids=out))
    model.check_numerics()
    model.close()
    torch.cuda.empty_cache()
    p_pre = p_dec = float("nan")
    if padded:
        print(f"[bench] padded to {L_max}, dense cache", file=sys.stderr, flush=True)
        pad = np.zeros((n, L_max), dtype=np.int32)
        for b, p in enumerate(prompts):
            pad[b, :len(p)] = p
        model = Q.Model(m, tensors, n, max_seq)
        pids = torch.from_numpy(pad).cuda()
        p_pre, p_dec = timed_runs(model, lambda out: model.prefill(pids, next_ids=out))
        model.close()
        torch.cuda.empty_cache()

    # algorithmic work of the ragged batch
    H, I, V, qd, kvd = m.hidden, m.intermediate, m.vocab, m.q_dim, m.kv_dim
    gemm_per_row = 2.0 * H * ((qd + 2 * kvd) + qd + 3 * I)
    attn = sum(2.0 * m.n_heads * m.head_dim * x * (x + 1) for x in lens)
    pflop = m.n_layers * (gemm_per_row * T + attn) + 2.0 * n * V * H
    e = 2
    weights = e * (m.n_layers * (H * (qd + 2 * kvd) + qd * H + 3 * H * I) + V * H)
    ctx_mean = T / n + (D - 1) / 2.0
    step_bytes = weights + n * m.n_layers * 2 * kvd * e * (ctx_mean + 1)
    return {
        "metric": "ragged batch on the paged KV cache vs the same prompts padded on the dense cache",
        "workload": f"{name}: Qwen2.5-1.5B shapes, bf16 weights, {n} prompts of {rw.min_len}..{rw.max_len} tokens "
                    f"(log-uniform, seed {rw.lens_seed}), {D} greedy decode steps",
        "prompt_tokens": T, "longest": L_max, "lengths": lens, "reps": reps,
        "ragged_paged": {"ttft_ms": round(r_pre, 3), "prefill_tokens_per_s": round(T / (r_pre / 1e3), 1),
                         "decode_ms_per_step": round(r_dec / D, 4), "decode_tokens_per_s": round(n * D / (r_dec / 1e3), 1),
                         "cache_blocks": n_blocks, "cache_bytes": n_blocks * blk * kv_elem_bytes},
        "padded_dense": {"ttft_ms": round(p_pre, 3), "prefill_tokens_per_s": round(T / (p_pre / 1e3), 1),
                         "decode_ms_per_step": round(p_dec / D, 4), "decode_tokens_per_s": round(n * D / (p_dec / 1e3), 1),
                         "cache_bytes": n * max_seq * kv_elem_bytes},
        "ttft_speedup": round(p_pre / r_pre, 2), "decode_speedup": round(p_dec / r_dec, 2),
        "decode_step_roofline": roof("hbm", "whole decode step, ragged (graph replay)",
                                     step_bytes / (r_dec / D / 1e3) / 1e9, HBM_PEAK_GBS, None, "GB/s",
                                     bytes_per_step=int(step_bytes)),
        "prefill_whole_roofline": roof("mfma", "whole ragged prefill (TTFT)", pflop / (r_pre / 1e3) / 1e12,
                                       MFMA_F16_PEAK_TFLOPS, None, "TFLOP/s", flop=pflop),
    }


def roof(bound, kernel, achieved, peak, measured_peak, unit, **extra):
    out = {"bound": bound, "kernel": kernel, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4)}
    if measured_peak:
        out["measured_peak"] = measured_peak
        out["frac_of_measured"] = round(achieved / measured_peak, 4)
    out.update(extra)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(S.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the in-run copy and MFMA peak measurements")
    ap.add_argument("--eager", action="store_true",
                    help="launch decode kernels one by one instead of replaying the captured graph "
                         "(same kernels; for counter collection, which does not follow graph launches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 4 device copies of 256 MiB (the reference for HBM byte counters)")
    ap.add_argument("--ragged", choices=sorted(S.RAGGED_WORKLOADS), default=None,
                    help="only compare a ragged batch on the paged cache with the same prompts padded on the "
                         "dense cache; prints its own JSON line")
    ap.add_argument("--no-padded", action="store_true", help="--ragged without the padded baseline")
    ap.add_argument("--cache-compare", type=int, default=0, metavar="STEPS",
                    help="only compare greedy generation of STEPS tokens with and without the KV cache "
                         "(qw_generate) on the workload's prompts; prints its own JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is "
              "a design only, not built", file=sys.stderr)
        sys.exit(2)

    import torch
    import decoder_only_transformer_qwen2_amd as Q

    if args.copy_calibration:
        # a plain copy of known size: the HBM counters of each dispatch read
        # 256 MiB fetched and 256 MiB written when the counters are exact
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": n, "dispatches": 4}), flush=True)
        return

    if args.ragged:
        print(json.dumps(ragged_compare(torch, Q, args.ragged, args.steps, args.warmup, not args.no_padded)),
              flush=True)
        return

    w = S.WORKLOADS[args.workload]
    m = w.model
    B, P, D = w.batch, w.prompt_len, w.decode_steps
    if args.cache_compare:
        print(json.dumps(cache_compare(torch, Q, w, args.cache_compare, args.steps, args.warmup)), flush=True)
        return
    peaks = None
    if not args.no_peaks:
        print("[bench] measured peaks (copy, MFMA)", file=sys.stderr, flush=True)
        peaks = measure_peaks(torch, Q)
    print(f"[bench] {args.workload}: generating weights", file=sys.stderr, flush=True)
    W = S.make_weights(m, w.weight_seed)
    ids_np = S.make_ids(w)
    model = Q.Model(m, Q.device_tensors(m, W), B, w.max_seq)
    torch.cuda.empty_cache()
    if args.eager:
        model.set_graph(False)
    ids = torch.from_numpy(ids_np).cuda()
    toks = torch.empty((D + 1, B), dtype=torch.int32, device="cuda")

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run_step(model, ids, toks, D, torch)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        run_step(model, ids, toks, D, torch, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prefill_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    decode_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    decode_tps = B * D / (decode_ms / 1e3)
    prefill_tps = B * P / (prefill_ms / 1e3)
    model.check_numerics()

    out = {"metric": METRIC, "value": round(decode_tps, 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16" if m.dtype == "bf16" else "f32",
           "data": "synthetic (seeded random-init weights N(0, 0.02) stored as bf16, uniform token ids)",
           "config": {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}", "batch": B, "prompt_len": P,
                      "decode_steps": D, "max_seq": w.max_seq,
                      "step": f"one prefill of {B} x {P} tokens + {D} greedy decode steps"},
           "prefill_tokens_per_s": round(prefill_tps, 1), "ttft_ms": round(prefill_ms, 3),
           "decode_ms_per_token_step": round(decode_ms / D, 4)}
    if peaks:
        out["measured_peaks"] = peaks
    # the decode step reads far more than it writes: the read-only pass is its ceiling
    hbm_meas = peaks["read_GBps"] if peaks else None
    mfma_meas = peaks["mfma_f16_TFLOPs"] if peaks else None

    if not args.no_roofline:
        # per-family decode time, each family timed over one eager pass
        fams = ["gemm_qkv", "rope_cache", "attention", "gemm_o", "gemm_gate_up", "gemm_down", "mlp", "attn_o",
                "attn_merge", "lm_head", "argmax", "rmsnorm", "embed"]
        per = {}
        for f in fams:
            model.prefill(ids, next_ids=toks[0])
            model.timing_enable(f)
            for s in range(D):
                model.decode_step(toks[s], next_ids=toks[s + 1])
            ms, n = model.timing_read(reset=True)
            model.timing_enable(None)
            per[f] = (ms, n)
        dom = max((f for f in per if per[f][1] > 0 and f in ("gemm_qkv", "attention", "gemm_o", "gemm_gate_up",
                                                               "gemm_down", "mlp", "attn_o", "lm_head")),
                  key=lambda f: per[f][0])
        ms, n = per[dom]
        avg_s = ms / n / 1e3
        ctx_mean = P + (D - 1) / 2.0
        bytes_per = decode_family_bytes(w, dom, ctx_mean)
        out["roofline"] = roof("hbm", dom, bytes_per / avg_s / 1e9, HBM_PEAK_GBS, hbm_meas, "GB/s",
                               traffic=measured_traffic(args.workload, dom), avg_launch_us=round(avg_s * 1e6, 3),
                               launches=n, algorithmic_bytes_per_launch=int(bytes_per))
        out["decode_family_ms_per_step"] = {f: round(per[f][0] / D, 4) for f in per}
        step_bytes = decode_step_bytes(w, ctx_mean)
        out["decode_step_roofline"] = roof("hbm", "whole decode step (graph replay)",
                                           step_bytes / (decode_ms / D / 1e3) / 1e9, HBM_PEAK_GBS, hbm_meas, "GB/s",
                                           bytes_per_step=int(step_bytes))
        # prefill: per-family time over one eager prefill each
        pper = {}
        for f in ("gemm_qkv", "attention", "gemm_o", "gemm_gate_up", "gemm_down", "rope_cache", "rmsnorm", "lm_head"):
            model.timing_enable(f)
            model.prefill(ids, next_ids=toks[0])
            ms, n = model.timing_read(reset=True)
            model.timing_enable(None)
            pper[f] = (ms, n)
        pdom = max(("gemm_qkv", "attention", "gemm_o", "gemm_gate_up", "gemm_down"), key=lambda f: pper[f][0])
        for key, f in (("prefill_roofline", pdom), ("prefill_attention_roofline", "attention")):
            ms, n = pper[f]
            tflops = prefill_family_flops(w, f) / (ms / n / 1e3) / 1e12
            out[key] = roof("mfma", f, tflops, MFMA_F16_PEAK_TFLOPS, mfma_meas, "TFLOP/s",
                            avg_launch_us=round(ms / n * 1e3, 3), launches=n,
                            flop_per_launch=prefill_family_flops(w, f))
        pflop = sum(prefill_family_flops(w, f) for f in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down",
                                                          "attention")) * m.n_layers
        pflop += prefill_family_flops(w, "lm_head")
        out["prefill_whole_roofline"] = roof("mfma", "whole prefill (TTFT)", pflop / (prefill_ms / 1e3) / 1e12,
                                             MFMA_F16_PEAK_TFLOPS, mfma_meas, "TFLOP/s", flop=pflop)
        out["prefill_family_ms"] = {f: round(pper[f][0], 3) for f in pper}

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, W, ids_np)
    model.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
