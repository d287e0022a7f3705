"""Brute-force route used to pin the oracle on tiny inputs.

Built differently from the oracle on purpose, so that a mistake in one is
unlikely to repeat in the other:
  * no KV cache: every generated position recomputes the whole prefix;
  * RoPE as an explicit hd x hd rotation matrix built from the pairwise
    (interleaved) block-diagonal definition of "LLM Speedrun: Architecture",
    section "Rotary Positional Embeddings RoPE", and then permuted into the
    split-half layout of section "Split-half RoPE implementation";
  * KV heads materialised per query head by repetition (section "Grouped Query
    Attention GQA": consecutive query heads share a KV head);
  * an explicit additive mask matrix and a textbook softmax written with
    Python loops over heads and rows;
  * every projection is an explicit sum over the [out, in] weight's rows.
Everything is float64.
"""
from __future__ import annotations

import math

import numpy as np


def decode(a):
    if a.dtype == np.uint16:
        return np.array([np.frombuffer(np.uint32(int(v) << 16).tobytes(), np.float32)[0]
                         for v in a.ravel()], dtype=np.float64).reshape(a.shape)
    return a.astype(np.float64)


def rotation_matrix(pos: int, hd: int, base: float) -> np.ndarray:
    """Split-half RoPE matrix for one position."""
    # pairwise definition: pair (2i, 2i+1) is turned by pos * base^(-2i/hd)
    Rp = np.zeros((hd, hd))
    for i in range(hd // 2):
        a = pos * base ** (-2.0 * i / hd)
        Rp[2 * i, 2 * i], Rp[2 * i, 2 * i + 1] = math.cos(a), -math.sin(a)
        Rp[2 * i + 1, 2 * i], Rp[2 * i + 1, 2 * i + 1] = math.sin(a), math.cos(a)
    # split-half keeps the real part of pair i at i and the imaginary part at i + hd/2
    perm = np.empty(hd, dtype=int)
    perm[0::2] = np.arange(hd // 2)
    perm[1::2] = np.arange(hd // 2) + hd // 2
    P = np.zeros((hd, hd))
    P[perm, np.arange(hd)] = 1.0            # P @ (interleaved vector) = split-half vector
    return P @ Rp @ P.T


def linear(x, W, b=None):
    out = np.zeros((x.shape[0], W.shape[0]))
    for o in range(W.shape[0]):
        out[:, o] = x @ W[o]
    if b is not None:
        out += b[None, :]
    return out


def norm(x, w, eps):
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        out[t] = x[t] / math.sqrt(float(np.sum(x[t] ** 2)) / x.shape[1] + eps) * w
    return out


def full_forward(shape, weights, ids):
    """Logits of every position of `ids` from scratch: [T, V]."""
    m = shape
    W = {k: decode(v) for k, v in weights.items()}
    T = len(ids)
    x = np.stack([W["model.embed_tokens.weight"][i] for i in ids])
    mask = np.zeros((T, T))
    for t in range(T):
        for s in range(T):
            if s > t:
                mask[t, s] = -1e9
    for l in range(m.n_layers):
        p = f"model.layers.{l}."
        u = norm(x, W[p + "input_layernorm.weight"], m.rms_eps)
        q = linear(u, W[p + "self_attn.q_proj.weight"], W[p + "self_attn.q_proj.bias"])
        k = linear(u, W[p + "self_attn.k_proj.weight"], W[p + "self_attn.k_proj.bias"])
        v = linear(u, W[p + "self_attn.v_proj.weight"], W[p + "self_attn.v_proj.bias"])
        q = q.reshape(T, m.n_heads, m.head_dim)
        k = k.reshape(T, m.n_kv_heads, m.head_dim)
        v = v.reshape(T, m.n_kv_heads, m.head_dim)
        for t in range(T):
            R = rotation_matrix(t, m.head_dim, m.rope_theta)
            q[t] = q[t] @ R.T
            k[t] = k[t] @ R.T
        g = m.n_heads // m.n_kv_heads
        k_rep = np.repeat(k, g, axis=1)
        v_rep = np.repeat(v, g, axis=1)
        o = np.zeros((T, m.n_heads, m.head_dim))
        for h in range(m.n_heads):
            scores = q[:, h, :] @ k_rep[:, h, :].T / math.sqrt(m.head_dim) + mask
            for t in range(T):
                row = scores[t]
                e = np.exp(row - row.max())
                o[t, h] = (e / e.sum()) @ v_rep[:, h, :]
        x = x + linear(o.reshape(T, -1), W[p + "self_attn.o_proj.weight"])
        u2 = norm(x, W[p + "post_attention_layernorm.weight"], m.rms_eps)
        gate = linear(u2, W[p + "mlp.gate_proj.weight"])
        up = linear(u2, W[p + "mlp.up_proj.weight"])
        x = x + linear(gate / (1.0 + np.exp(-gate)) * up, W[p + "mlp.down_proj.weight"])
    y = norm(x, W["model.norm.weight"], m.rms_eps)
    return linear(y, W["model.embed_tokens.weight"])


def generate(shape, weights, prompt, steps):
    """Greedy generation with no cache: each step re-runs the whole prefix."""
    seq = list(prompt)
    toks, logits = [], []
    for _ in range(steps + 1):
        lg = full_forward(shape, weights, seq)[-1]
        logits.append(lg)
        best = 0
        for i in range(1, len(lg)):
            if lg[i] > lg[best]:
                best = i
        toks.append(best)
        seq.append(best)
    return np.array(toks), np.stack(logits)
