"""Throughput of the Qwen2 decoder forward on one MI355X.

A step is one pass of the whole hot path over one batch: prefill of the
batch's prompts (the TTFT token), then the workload's greedy decode steps,
each through the C ABI of libqw.so.  Inputs (weights, token ids) are seeded
synthetic data resident in HBM before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 0.5b]

Prints one JSON line.  `value` is decode tokens/s over the timed steps;
prefill tokens/s and TTFT ride along.  `roofline` covers the kernel family
with the most decode time, timed with HIP events on the model's stream over
an extra, eagerly launched pass (same kernels, same data); `cpu_baseline` is
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
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
# committed rocprofv3 counter summary for the dominant decode kernel
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dec_mlp_0.5b_hbm_traffic.json")
MFMA_F16_PEAK_TFLOPS = 2500.0
DESCRIPTIONS = {
    "tiny": "tiny Qwen2-style decoder, fp32 (2 layers, hidden 128), batch 1, prompt 16, 8 greedy decode steps",
    "0.5b": "Qwen2.5-0.5B shapes, bf16 weights, batch 1, prompt 128, 128 greedy decode steps, cache 2048",
    "1.5b": "Qwen2.5-1.5B shapes, bf16 weights, batch 1, prompt 512, 256 greedy decode steps, cache 1024",
    "1.5b-prefill": "Qwen2.5-1.5B shapes, bf16 weights, batch 8 x prompt 2048, 32 greedy decode steps, cache 4096",
    "1.5b-longctx": "Qwen2.5-1.5B shapes, bf16 weights, batch 32 x prompt 8192, 128 greedy decode steps, cache 8320",
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


def measured_traffic(workload: str, family: str):
    """HBM bytes per launch of a kernel family from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads for
    a copy of known size), or None when the summary is for another workload or
    family, or the kernel's source file has changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
        with open(os.path.join(ROOT, d["kernel_source"]), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError, KeyError):
        return None
    if sha != d.get("kernel_source_sha256") or d.get("workload") != workload or d.get("family") != family:
        return None
    return int(d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"])


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


def cpu_baseline(w: S.Workload, W, ids, budget_s: float = 15.0):
    """The oracle, untuned, on batch row 0: prefill, then decode steps until
    the time budget is spent.  Reports decode tokens/s of the sample."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    om = O.OracleModel(w.model, W)
    cache = om.new_cache(w.prompt_len + w.decode_steps)
    t0 = time.perf_counter()
    lg = om.forward(ids[0], 0, cache)
    t_prefill = time.perf_counter() - t0
    tok = O.greedy_token(lg)
    n, t1 = 0, time.perf_counter()
    while n < w.decode_steps and (time.perf_counter() - t1) < budget_s:
        lg = om.forward([tok], w.prompt_len + n, cache)
        tok = O.greedy_token(lg)
        n += 1
    t_dec = time.perf_counter() - t1
    return {"value": round(n / t_dec, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"batch row 0 of {w.batch}: prefill of {w.prompt_len} tokens "
                      f"({w.prompt_len / t_prefill:.1f} tokens/s, TTFT {t_prefill * 1e3:.0f} ms), "
                      f"then the first {n} decode steps (fp64 numpy oracle)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="0.5b", choices=sorted(S.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch decode kernels one by one instead of replaying the captured graph "
                         "(same kernels; for counter collection, which does not follow graph launches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 4 device copies of 256 MiB (the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is "
              "described in DESIGN.md but not built", file=sys.stderr)
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

    w = S.WORKLOADS[args.workload]
    m = w.model
    B, P, D = w.batch, w.prompt_len, w.decode_steps
    print(f"[bench] {args.workload}: generating weights", file=sys.stderr, flush=True)
    W = S.make_weights(m, w.weight_seed)
    ids_np = S.make_ids(w)
    model = Q.Model(m, Q.device_tensors(m, W), B, w.max_seq)
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

    out = {"metric": METRIC, "value": round(decode_tps, 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16" if m.dtype == "bf16" else "f32",
           "data": "synthetic (seeded random-init weights N(0, 0.02), uniform token ids)",
           "config": {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}", "batch": B, "prompt_len": P,
                      "decode_steps": D, "max_seq": w.max_seq},
           "prefill_tokens_per_s": round(prefill_tps, 1), "ttft_ms": round(prefill_ms, 3),
           "decode_ms_per_token_step": round(decode_ms / D, 4)}

    if not args.no_roofline:
        # per-family decode time, each family timed over one eager pass
        fams = ["gemm_qkv", "rope_cache", "attention", "gemm_o", "gemm_gate_up", "gemm_down", "mlp", "attn_o", "attn_merge", "lm_head",
                "argmax", "rmsnorm", "embed"]
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
        achieved = bytes_per / avg_s / 1e9
        out["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic(args.workload, dom),
                           "avg_launch_us": round(avg_s * 1e6, 3), "launches": n,
                           "algorithmic_bytes_per_launch": int(bytes_per)}
        out["decode_family_ms_per_step"] = {f: round(per[f][0] / D, 4) for f in per}
        step_gbs = decode_step_bytes(w, ctx_mean) / (decode_ms / D / 1e3) / 1e9
        out["decode_step_roofline"] = {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                                       "bytes_per_step": int(decode_step_bytes(w, ctx_mean))}
        # prefill: per-family time over one eager prefill each
        pper = {}
        for f in ("gemm_qkv", "attention", "gemm_o", "gemm_gate_up", "gemm_down", "rope_cache", "rmsnorm", "lm_head"):
            model.timing_enable(f)
            model.prefill(ids, next_ids=toks[0])
            ms, n = model.timing_read(reset=True)
            model.timing_enable(None)
            pper[f] = (ms, n)
        pdom = max(("gemm_qkv", "attention", "gemm_o", "gemm_gate_up", "gemm_down"), key=lambda f: pper[f][0])
        ms, n = pper[pdom]
        tflops = prefill_family_flops(w, pdom) / (ms / n / 1e3) / 1e12
        out["prefill_roofline"] = {"bound": "mfma", "kernel": pdom, "achieved": round(tflops, 1),
                                   "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                                   "avg_launch_us": round(ms / n * 1e3, 3), "launches": n}
        out["prefill_family_ms"] = {f: round(pper[f][0], 3) for f in pper}

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, W, ids_np)
    model.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
