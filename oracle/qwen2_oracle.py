"""CPU oracle for the Qwen2.5 decoder forward: prefill and KV-cached greedy decode.

TEST INFRASTRUCTURE.  This is a plain, slow, obviously-correct restatement of
what the decoder computes, used only to check the HIP library.  Only the test
suite, `__graft_entry__.smoke()` and the `cpu_baseline` leg of `bench.py` may
import it; the product path never does, and it shares no code with the HIP
library (the two meet only in the seeded inputs of `synthetic`).

Precision: every value is float64.  Weights are read exactly (bf16 storage is
the top half of an IEEE float32; see `decode_storage`).  No activation is
rounded to bf16: the oracle is the real-valued forward pass of the given
weights, so it is the same reference for the library's fp32, bf16 and fp16
weight modes.

Layout: rows are tokens, so activations are [T, features] and a projection
with an HF-layout weight W [out, in] is `u @ W.T`.

Sources, cited by page title and section:
  [A]  "augur" -- feature list: RMSNorm before attention, before the MLP and
       after the last layer; RoPE on q and k; grouped-query attention; causal
       masking; SwiGLU MLP; pre-norm blocks; embeddings -> layers -> final norm
       -> LM head; greedy generation; prefill/decode split; preallocated KV cache.
  [S]  "LLM Speedrun: Architecture" -- sections "Attention", "What's up with
       Softmax?", "Every token with every other token, even the future ones?",
       "Normalization", "Why pre-norm over post-norm?", "Multi Head Attention",
       "Grouped Query Attention GQA", "Rotary Positional Embeddings RoPE",
       "Split-half RoPE implementation", "Decoding", "Introducing bias", and
       its harness listing (bf16 -> f32 reading, the GQA / SwiGLU / RMSNorm
       classes and the generation loop).
  [B]  "Building a Qwen2.5-1.5B Inference Engine From Scratch" -- section 1
       (prefill populates the KV cache, decode feeds one token at a time) and
       section 1.1 (compare logits, not only tokens).

Readings where the pages are silent:
  * RoPE angle pos * theta**(-2i/hd) is evaluated in float64 (the harness
    listing evaluates it in float32; exact evaluation is the plain reading of
    the formula).
  * The mask value -1e9 of the listing is taken as "masked keys get zero
    weight", which is what -1e9 does after exp in any float format.
  * Greedy choice is the lowest index among equal maxima (numpy argmax rule).
  * q/k/v projections carry a bias; o_proj, gate, up, down and the head don't.
"""
from __future__ import annotations

import os
from typing import Dict, Optional

import numpy as np

__all__ = [
    "decode_storage", "rms_norm", "rope_inverse_frequencies", "rope_rotate",
    "attention_weights", "causal_gqa_attention", "silu", "swiglu_mlp",
    "greedy_token", "philox4x64_10", "sampling_draw", "sample_token", "OracleModel",
]


# ---------------------------------------------------------------- reading weights
def decode_storage(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of stored weights.  [S] harness listing's tensor
    reader: a bf16 word is the high 16 bits of a float32, so shifting it left
    by 16 and reinterpreting gives the value exactly.  float16 and float32
    widen exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float16, np.float32, np.float64):
        return a.astype(np.float64)
    raise ValueError(f"unsupported weight storage dtype {a.dtype}")


# ---------------------------------------------------------------- building blocks
def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """[S] "Normalization" and the listing's RMSNorm; [A] RMSNorm.  Each row is
    divided by the root of (mean of its squares + eps), then scaled by w."""
    mean_sq = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(mean_sq + eps) * w


def rope_inverse_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """[S] "Rotary Positional Embeddings RoPE": pair i rotates at frequency
    theta**(-2i/d), i = 0 .. d/2-1, with d the head dimension."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * i / head_dim)


def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Split-half RoPE, [S] "Split-half RoPE implementation": within each head
    of x [T, heads, hd], element i of the first half is the real part and
    element i + hd/2 the imaginary part of one complex number, which is turned
    by the angle pos * freq_i.  A rotation by a of (re, im) gives
    (re cos a - im sin a, im cos a + re sin a)."""
    hd = x.shape[-1]
    half = hd // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_inverse_frequencies(hd, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    re, im = x[..., :half], x[..., half:]
    return np.concatenate([re * c - im * s, im * c + re * s], axis=-1)


def attention_weights(q: np.ndarray, k: np.ndarray, q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """One head: [S] "Attention" (scores q.k / sqrt(d_k)), "What's up with
    Softmax?" (max-subtracted softmax over keys) and "Every token with every
    other token" (a query at position p sees only keys at positions <= p).
    q [T, hd], k [S, hd] -> probabilities [T, S]; masked entries are 0.
    (Each step works in place on the one [T, S] array: the same values as
    fresh arrays per step, without allocating several of them at long
    contexts.)"""
    scores = q @ k.T
    scores /= np.sqrt(q.shape[-1])
    hidden = k_pos[None, :] > q_pos[:, None]
    scores[hidden] = -np.inf
    scores -= scores.max(axis=-1, keepdims=True)
    np.exp(scores, out=scores)
    scores /= scores.sum(axis=-1, keepdims=True)
    return scores


# Query rows per block in causal_gqa_attention.
_ROWS_PER_BLOCK = 512


def causal_gqa_attention(q, k, v, q_pos, k_pos):
    """[S] "Grouped Query Attention GQA" / [A] grouped-query attention: query
    head h reads KV head floor(h / g), g = n_heads / n_kv_heads (consecutive
    query heads share one KV head, as repeating each KV head g times does).
    q [T, nq, hd]; k, v [S, nkv, hd] -> [T, nq, hd].

    Evaluation order only (no arithmetic changes): every output row depends
    on its own query row alone, so rows are taken in blocks, and a block
    meets only the keys at or before its last row's position (k_pos must be
    ascending); any key past that is masked for every row of the block and
    would get weight exactly 0.  Heads are independent and run on a thread
    pool, with the matrix library single-threaded inside each head."""
    nq, nkv = q.shape[1], k.shape[1]
    g = nq // nkv
    k_pos = np.asarray(k_pos)
    q_pos = np.asarray(q_pos)
    if k_pos.size > 1 and np.any(np.diff(k_pos) <= 0):
        raise ValueError("key positions must be ascending")
    out = np.empty(q.shape, dtype=np.float64)

    def one_head(h):
        j = h // g
        for a in range(0, q.shape[0], _ROWS_PER_BLOCK):
            b = min(a + _ROWS_PER_BLOCK, q.shape[0])
            n_keys = int(np.searchsorted(k_pos, q_pos[a:b].max(), side="right"))
            p = attention_weights(q[a:b, h, :], k[:n_keys, j, :], q_pos[a:b], k_pos[:n_keys])
            out[a:b, h, :] = p @ v[:n_keys, j, :]

    work = q.shape[0] * k.shape[0]
    if nq == 1 or work < (1 << 22):
        for h in range(nq):
            one_head(h)
        return out
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    threads = max(1, min(nq, len(os.sched_getaffinity(0))))
    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        list(ex.map(one_head, range(nq)))
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """[S] listing's swish: z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_mlp(u, w_gate, w_up, w_down):
    """[S] "But how does it remember things?" and the listing's SwiGLU FFN;
    [A] Qwen MLP: down( silu(gate u) * (up u) )."""
    return (silu(u @ w_gate.T) * (u @ w_up.T)) @ w_down.T


def greedy_token(logits: np.ndarray) -> int:
    """[A] greedy generation / [S] decoder step: the index of the largest
    logit; among equal maxima, the lowest index."""
    return int(np.argmax(logits))


# ---------------------------------------------------------------- sampling
# "augur" lists temperature, top-k and top-p sampling as not yet built; the
# pages give no formulas for them, so the plain reading is taken: keep the
# top_k largest logits (ties: lower index first), weight
# them by exp((l - l_max) / temperature), keep the shortest prefix of that
# order whose weight reaches top_p of the total, and pick by the inverse
# cumulative distribution of one uniform draw u in [0, 1).

_M64 = (1 << 64) - 1


def philox4x64_10(counter, key):
    """Philox-4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel
    random numbers: as easy as 1, 2, 3", SC 2011): each round multiplies
    words 0 and 2 by the two round multipliers, crosses the high halves with
    words 1 and 3 and the key, and the key is bumped by the two Weyl
    constants between rounds.  counter: 4 ints, key: 2 ints (each < 2^64)."""
    c = [int(x) & _M64 for x in counter]
    k = [int(x) & _M64 for x in key]
    for _ in range(10):
        p0 = 0xD2E7470EE14C6C93 * c[0]
        p1 = 0xCA5A826395121157 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & _M64, (p0 >> 64) ^ c[3] ^ k[1], p0 & _M64]
        k = [(k[0] + 0x9E3779B97F4A7C15) & _M64, (k[1] + 0xBB67AE8584CAA73B) & _M64]
    return c


def sampling_draw(seed: int, sequence: int, n: int) -> float:
    """The uniform draw for the token that follows the first n tokens of
    batch row `sequence`: the top 24 bits of the first Philox word of counter
    (n, sequence, 0, 0) under key (seed, 0), as a multiple of 2^-24."""
    w = philox4x64_10([n, sequence, 0, 0], [seed, 0])[0]
    return (w >> 40) * 2.0 ** -24


def sample_token(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float):
    """The sampled index and the cumulative weights it was chosen from
    (float64): (token, candidates in order, cumulative weights C, kept m,
    threshold r = u * C[m-1]).  The token is the first kept candidate j with
    C[j] > r."""
    logits = np.asarray(logits, dtype=np.float64)
    order = np.lexsort((np.arange(logits.size), -logits))[:top_k]   # value desc, index asc
    w = np.exp((logits[order] - logits[order[0]]) / temperature)
    C = np.cumsum(w)
    m = int(np.searchsorted(C, top_p * C[-1], side="left")) + 1
    m = min(max(m, 1), len(C))
    r = u * C[m - 1]
    j = int(np.searchsorted(C[:m], r, side="right"))
    return int(order[min(j, m - 1)]), order, C, m, r


# ---------------------------------------------------------------- the model
class OracleModel:
    """Qwen2 decoder of one sequence at a time (batch rows never interact).

    `weights` maps HF parameter names to stored arrays ([out, in] layout).
    The KV cache is a preallocated pair of arrays per layer, [A] "Preallocated
    KV-cache"; a forward over ids at positions start .. start+T-1 writes their
    keys and values at those positions and attends over 0 .. start+T-1.
    """

    def __init__(self, shape, weights: Dict[str, np.ndarray]):
        self.m = shape
        W = {k: decode_storage(v) for k, v in weights.items()}
        self.embed = W["model.embed_tokens.weight"]                      # [V, H]
        self.head = W.get("lm_head.weight", self.embed)                  # tied
        self.final_norm = W["model.norm.weight"]
        self.layers = []
        for l in range(shape.n_layers):
            p = f"model.layers.{l}."
            self.layers.append({k: W[p + k] for k in (
                "input_layernorm.weight", "post_attention_layernorm.weight",
                "self_attn.q_proj.weight", "self_attn.q_proj.bias",
                "self_attn.k_proj.weight", "self_attn.k_proj.bias",
                "self_attn.v_proj.weight", "self_attn.v_proj.bias",
                "self_attn.o_proj.weight",
                "mlp.gate_proj.weight", "mlp.up_proj.weight", "mlp.down_proj.weight")})

    # -- cache
    def new_cache(self, max_seq: int):
        m = self.m
        return {"k": np.zeros((m.n_layers, max_seq, m.n_kv_heads, m.head_dim)),
                "v": np.zeros((m.n_layers, max_seq, m.n_kv_heads, m.head_dim)),
                "len": 0}

    # -- one decoder block, [S] "Why pre-norm over post-norm?" / [A] decoder blocks
    def _block(self, l: int, x: np.ndarray, start: int, cache) -> np.ndarray:
        m, lw = self.m, self.layers[l]
        T = x.shape[0]
        pos = np.arange(start, start + T)
        u = rms_norm(x, lw["input_layernorm.weight"], m.rms_eps)
        q = u @ lw["self_attn.q_proj.weight"].T + lw["self_attn.q_proj.bias"]
        k = u @ lw["self_attn.k_proj.weight"].T + lw["self_attn.k_proj.bias"]
        v = u @ lw["self_attn.v_proj.weight"].T + lw["self_attn.v_proj.bias"]
        q = rope_rotate(q.reshape(T, m.n_heads, m.head_dim), pos, m.rope_theta)
        k = rope_rotate(k.reshape(T, m.n_kv_heads, m.head_dim), pos, m.rope_theta)
        v = v.reshape(T, m.n_kv_heads, m.head_dim)
        cache["k"][l, start:start + T] = k
        cache["v"][l, start:start + T] = v
        S = start + T
        o = causal_gqa_attention(q, cache["k"][l, :S], cache["v"][l, :S], pos, np.arange(S))
        x = x + o.reshape(T, m.q_dim) @ lw["self_attn.o_proj.weight"].T
        u2 = rms_norm(x, lw["post_attention_layernorm.weight"], m.rms_eps)
        return x + swiglu_mlp(u2, lw["mlp.gate_proj.weight"], lw["mlp.up_proj.weight"],
                              lw["mlp.down_proj.weight"])

    def forward(self, ids, start: int, cache, logits_rows: Optional[slice] = None, progress=None) -> np.ndarray:
        """Tokens `ids` at positions start.., given a cache holding 0..start-1.
        Returns logits [V] of the last row, or [rows, V] for `logits_rows`
        ([A] full forward pass: embeddings, layers, final norm, LM head).
        `progress`, if given, is called with each finished layer's index."""
        ids = np.asarray(ids, dtype=np.int64).reshape(-1)
        if start != cache["len"]:
            raise ValueError("forward must continue the cached sequence")
        x = self.embed[ids]                                              # [T, H]
        for l in range(self.m.n_layers):
            x = self._block(l, x, start, cache)
            if progress:
                progress(l)
        cache["len"] = start + len(ids)
        rows = x[-1:] if logits_rows is None else x[logits_rows]
        y = rms_norm(rows, self.final_norm, self.m.rms_eps)
        logits = y @ self.head.T
        return logits[0] if logits_rows is None else logits

    # -- the generation loop, [B] section 1 and [A] prefill/decode split
    def generate(self, prompt, steps: int, max_seq: Optional[int] = None):
        """Prefill, then `steps` cached decode steps.  Returns the steps+1
        greedy tokens and their logits [steps+1, V]."""
        prompt = list(np.asarray(prompt).reshape(-1))
        cache = self.new_cache(max_seq or len(prompt) + steps)
        logits = [self.forward(prompt, 0, cache)]
        toks = [greedy_token(logits[-1])]
        for s in range(steps):
            logits.append(self.forward([toks[-1]], len(prompt) + s, cache))
            toks.append(greedy_token(logits[-1]))
        return np.array(toks), np.stack(logits)

    def teacher_forced(self, prompt, fed, progress=None) -> np.ndarray:
        """Logits after the prompt and after each token of `fed` (the ids a
        decoder emitted), from one uncached forward over prompt + fed:
        [len(fed) + 1, V].  By causality row i equals what a cached decode
        that was fed the same ids would produce at that step."""
        prompt = list(np.asarray(prompt).reshape(-1))
        fed = list(np.asarray(fed).reshape(-1))
        seq = prompt + fed
        cache = self.new_cache(len(seq))
        return self.forward(seq, 0, cache, logits_rows=slice(len(prompt) - 1, len(seq)), progress=progress)
