"""Shared pieces of the parity tests: running the HIP library through its
C ABI, and the teacher-forced comparison against the CPU oracle."""
from __future__ import annotations

import numpy as np

import synthetic as S

# Tolerances: max |logit_gpu - logit_oracle| per step, and the oracle's top-2
# margin above which the greedy token must match exactly.  The bf16-weight
# mode computes with fp16 operands and fp32 accumulation; fp32 mode is fp32
# throughout.
LOGIT_TOL = {"f32": 1e-3, "bf16": 5e-2, "f16": 5e-2}
TOKEN_MARGIN = 0.1
# fp32 mode is also held to exact tokens wherever the margin exceeds twice the
# logit tolerance (a flip there would need an error above the tolerance).
F32_STRICT_MARGIN = 2e-3


def with_random_norms(W, m, seed=21):
    """Norm weights drawn around 1 (the synthetic init sets them to exactly 1,
    which would hide a dropped norm-weight multiply)."""
    rng = np.random.default_rng(seed)
    W = dict(W)
    for k in W:
        if k.endswith("layernorm.weight") or k == "model.norm.weight":
            f = (1.0 + 0.3 * rng.standard_normal(W[k].shape)).astype(np.float32)
            W[k] = (S.f32_to_bf16_bits(f) if W[k].dtype == np.uint16
                    else f.astype(W[k].dtype))
    return W


def gpu_generate(model, ids_np, steps, want_logits=True, graph=True):
    """Prefill + `steps` decode steps through the C ABI.  Returns tokens
    [B, steps+1] and (optionally) logits [B, steps+1, V] as numpy."""
    import torch
    B, P = ids_np.shape
    V = model.shape.vocab
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    model.set_graph(graph)
    toks = torch.empty((steps + 1, B), dtype=torch.int32, device="cuda")
    logits = torch.empty((steps + 1, B, V), dtype=torch.float32, device="cuda") if want_logits else None
    model.prefill(ids, logits=logits[0] if want_logits else None, next_ids=toks[0])
    for s in range(steps):
        model.decode_step(toks[s], logits=logits[s + 1] if want_logits else None, next_ids=toks[s + 1])
    torch.cuda.synchronize()
    t = toks.cpu().numpy().T.copy()
    lg = logits.permute(1, 0, 2).cpu().numpy() if want_logits else None
    return t, lg


def compare_row(oracle_model, prompt, gpu_tokens, gpu_logits, dtype, label="", ref=None):
    """Teacher-forced check of one sequence: the oracle is fed the GPU's own
    token stream, so every step is compared on the same prefix.  `ref` may
    hold the oracle's teacher-forced logits when the caller has them."""
    if ref is None:
        ref = oracle_model.teacher_forced(prompt, gpu_tokens[:-1])
    err = np.abs(gpu_logits.astype(np.float64) - ref)
    per_step = err.max(axis=1)
    tol = LOGIT_TOL[dtype]
    assert np.all(np.isfinite(gpu_logits)), f"{label}: non-finite GPU logits"
    assert per_step.max() <= tol, f"{label}: max |dlogit| {per_step.max():.3e} > {tol} (per step {per_step})"
    srt = np.sort(ref, axis=1)
    margin = srt[:, -1] - srt[:, -2]
    oracle_tok = ref.argmax(axis=1)
    need = margin > (F32_STRICT_MARGIN if dtype == "f32" else TOKEN_MARGIN)
    bad = np.nonzero(need & (oracle_tok != gpu_tokens))[0]
    assert bad.size == 0, f"{label}: token mismatch at steps {bad} (margins {margin[bad]})"
    return per_step.max(), int(need.sum())


def assert_same_sequence(t_a, l_a, t_b, l_b, tol=2e-2, label=""):
    """Two free-running GPU generations of one sequence under different launch
    shapes (batch sizes pick different split counts and norm placement, so
    rounding order differs).  Up to the first step where their tokens differ
    the two runs see the same prefix: logits must agree within `tol`.  At that
    step the choice must have been a near-tie (top-2 margin <= 2 * tol) --
    after it the runs decode different sequences and are not compared.
    Rows leaking into each other would differ by O(1) before any divergence."""
    n = len(t_a)
    diff_steps = np.nonzero(t_a != t_b)[0]
    k = int(diff_steps[0]) if diff_steps.size else n - 1
    d = np.abs(l_a[:k + 1].astype(np.float64) - l_b[:k + 1]).max()
    assert d <= tol, f"{label}: max |dlogit| between runs over steps 0..{k}: {d:.3e} > {tol}"
    if diff_steps.size:
        srt = np.sort(l_a[k])
        margin = float(srt[-1] - srt[-2])
        assert margin <= 2 * tol, f"{label}: tokens differ at step {k} with a clear margin {margin:.3e}"
    return d
