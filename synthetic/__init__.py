"""Seeded synthetic inputs shared by the oracle and the GPU path.

This module only *describes and draws* inputs: model shapes, run shapes,
random-init weights and random token ids.  It holds none of the decoder's
arithmetic, so the CPU oracle and the HIP library can both consume the same
buffers without sharing any computation.

Workload shapes follow the Qwen2.5 model cards the pages discuss ("Building a
Qwen2.5-1.5B Inference Engine From Scratch", section 1.1: 28 layers, 12 query
heads, 2 KV heads, 1,543,714,304 parameters) and the Qwen2-style config fields
the "augur" page lists (hidden size, head counts, MLP size, RMSNorm epsilon,
RoPE theta, vocabulary size).

Drawing rule (one reading, since the pages fix no seeds):
  * every tensor gets its own numpy stream, SeedSequence([seed, tensor_index]),
    tensor_index counting in the order of `tensor_names(cfg)`;
  * non-norm tensors (projection weights, q/k/v biases, the embedding) are
    float32 standard normals times 0.02; norm weights are exactly 1;
  * bf16 models store the nearest bf16 (round-to-nearest-even) of that draw,
    as raw uint16 bit patterns; fp16 models the nearest float16; fp32 models
    the float32 draw;
  * token ids are uniform integers in [0, vocab) from default_rng(seed + 1).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

__all__ = [
    "ModelShape", "Workload", "WORKLOADS", "MODEL_SHAPES", "RaggedWorkload", "RAGGED_WORKLOADS", "tensor_names",
    "tensor_shape", "make_weights", "make_ids", "param_count", "f32_to_bf16_bits",
]


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Qwen2-style decoder shape.  Field names follow the HF config keys."""
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    dtype: str = "bf16"          # weight storage: "bf16", "f16" or "f32"
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    qkv_bias: bool = True
    tie_embeddings: bool = True

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    """A model shape plus a run: batch x prompt, then `decode_steps` greedy
    steps, with a KV cache of `max_seq` positions per sequence."""
    name: str
    model: ModelShape
    batch: int
    prompt_len: int
    decode_steps: int
    max_seq: int
    weight_seed: int = 0

    @property
    def ids_seed(self) -> int:
        return self.weight_seed + 1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY = ModelShape("tiny-qwen2", n_layers=2, hidden=128, n_heads=4, n_kv_heads=2,
                  head_dim=32, intermediate=384, vocab=1024, dtype="f32")
QWEN25_05B = ModelShape("qwen2.5-0.5b", n_layers=24, hidden=896, n_heads=14, n_kv_heads=2,
                        head_dim=64, intermediate=4864, vocab=151936)
QWEN25_15B = ModelShape("qwen2.5-1.5b", n_layers=28, hidden=1536, n_heads=12, n_kv_heads=2,
                        head_dim=128, intermediate=8960, vocab=151936)

# Qwen2.5-Coder-7B ("LLM Speedrun: Architecture", "Plugging in the specific
# parameters" and the harness listing's config): 28/4 heads of 128, a
# separate (untied) LM head over a 152064-entry vocabulary.
QWEN25_CODER_7B = ModelShape("qwen2.5-coder-7b", n_layers=28, hidden=3584, n_heads=28, n_kv_heads=4,
                             head_dim=128, intermediate=18944, vocab=152064, tie_embeddings=False)

MODEL_SHAPES = {m.name: m for m in (TINY, QWEN25_05B, QWEN25_15B, QWEN25_CODER_7B)}

# The five workloads.  The 1.5B runs leave the cache size open; the readings
# are 1024 for the 512+256 run and 8192+128 = 8320 for the long-context run.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, batch=1, prompt_len=16, decode_steps=8, max_seq=64),
    "0.5b": Workload("0.5b", QWEN25_05B, batch=1, prompt_len=128, decode_steps=128, max_seq=2048),
    "1.5b": Workload("1.5b", QWEN25_15B, batch=1, prompt_len=512, decode_steps=256, max_seq=1024),
    "1.5b-prefill": Workload("1.5b-prefill", QWEN25_15B, batch=8, prompt_len=2048,
                             decode_steps=32, max_seq=4096),
    "1.5b-longctx": Workload("1.5b-longctx", QWEN25_15B, batch=32, prompt_len=8192,
                             decode_steps=128, max_seq=8320),
    # the second model family the pages name (not one of the five graded
    # workloads): one sequence, as the speedrun harness runs it
    "coder-7b": Workload("coder-7b", QWEN25_CODER_7B, batch=1, prompt_len=512, decode_steps=128, max_seq=1024),
}


@dataclasses.dataclass(frozen=True)
class RaggedWorkload:
    """A batch of prompts of different lengths (ragged, no padding): n
    lengths drawn log-uniformly from [min_len, max_len] (seeded), then
    `decode_steps` greedy steps; a paged cache sized to the positions held."""
    name: str
    model: ModelShape
    n: int
    min_len: int
    max_len: int
    decode_steps: int
    weight_seed: int = 0
    lens_seed: int = 7

    def lengths(self) -> List[int]:
        rng = np.random.default_rng(self.lens_seed)
        u = rng.random(self.n)
        lens = np.exp(np.log(self.min_len) + u * (np.log(self.max_len) - np.log(self.min_len)))
        return [int(min(self.max_len, max(self.min_len, round(x)))) for x in lens]

    def prompts(self) -> List[np.ndarray]:
        rng = np.random.default_rng(self.weight_seed + 1)
        return [rng.integers(0, self.model.vocab, n, dtype=np.int64).astype(np.int32) for n in self.lengths()]


# Ragged serving batch (the pages' "not yet" list: paged attention, batches
# of prompts of different lengths): 32 prompts of 256 .. 8192 tokens.
RAGGED_WORKLOADS: Dict[str, RaggedWorkload] = {
    "1.5b-ragged": RaggedWorkload("1.5b-ragged", QWEN25_15B, n=32, min_len=256, max_len=8192, decode_steps=128),
}

_LAYER_TENSORS = (
    "input_layernorm.weight",
    "self_attn.q_proj.weight", "self_attn.q_proj.bias",
    "self_attn.k_proj.weight", "self_attn.k_proj.bias",
    "self_attn.v_proj.weight", "self_attn.v_proj.bias",
    "self_attn.o_proj.weight",
    "post_attention_layernorm.weight",
    "mlp.gate_proj.weight", "mlp.up_proj.weight", "mlp.down_proj.weight",
)


def tensor_names(m: ModelShape) -> List[str]:
    """HF Qwen2 parameter names in generation order (tied head: no lm_head)."""
    names = ["model.embed_tokens.weight"]
    for l in range(m.n_layers):
        names += [f"model.layers.{l}.{t}" for t in _LAYER_TENSORS]
    names.append("model.norm.weight")
    if not m.tie_embeddings:
        names.append("lm_head.weight")
    return names


def tensor_shape(m: ModelShape, name: str):
    """[out, in] shapes as the HF checkpoints store them."""
    H, I, V = m.hidden, m.intermediate, m.vocab
    leaf = name.split("model.layers.")[-1].split(".", 1)[-1] if "layers." in name else name
    table = {
        "model.embed_tokens.weight": (V, H), "lm_head.weight": (V, H), "model.norm.weight": (H,),
        "input_layernorm.weight": (H,), "post_attention_layernorm.weight": (H,),
        "self_attn.q_proj.weight": (m.q_dim, H), "self_attn.q_proj.bias": (m.q_dim,),
        "self_attn.k_proj.weight": (m.kv_dim, H), "self_attn.k_proj.bias": (m.kv_dim,),
        "self_attn.v_proj.weight": (m.kv_dim, H), "self_attn.v_proj.bias": (m.kv_dim,),
        "self_attn.o_proj.weight": (H, m.q_dim),
        "mlp.gate_proj.weight": (I, H), "mlp.up_proj.weight": (I, H),
        "mlp.down_proj.weight": (H, I),
    }
    return table[leaf]


def param_count(m: ModelShape) -> int:
    return int(sum(int(np.prod(tensor_shape(m, n))) for n in tensor_names(m)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of float32 values, as uint16 bit patterns.
    NaN stays NaN (quiet); the draws here are always finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def _draw(m: ModelShape, name: str, index: int, seed: int) -> np.ndarray:
    shape = tensor_shape(m, name)
    if name.endswith("layernorm.weight") or name == "model.norm.weight":
        f = np.ones(shape, dtype=np.float32)
    else:
        rng = np.random.default_rng(np.random.SeedSequence([seed, index]))
        f = rng.standard_normal(size=shape, dtype=np.float32)
        f *= np.float32(0.02)
    if m.dtype == "bf16":
        return f32_to_bf16_bits(f)
    if m.dtype == "f16":
        return f.astype(np.float16)                  # nearest fp16 (ties to even)
    return f


def make_weights(m: ModelShape, seed: int = 0, only=None) -> Dict[str, np.ndarray]:
    """Seeded random-init weights keyed by HF name.  bf16 models give uint16
    bit patterns, fp32 models give float32.  `only` restricts the names drawn
    (each tensor's stream depends only on (seed, index), so subsets agree)."""
    out = {}
    for i, name in enumerate(tensor_names(m)):
        if only is not None and name not in only:
            continue
        out[name] = _draw(m, name, i, seed)
    return out


def make_ids(w: Workload) -> np.ndarray:
    """Prompt token ids [batch, prompt_len], int32, uniform in [0, vocab)."""
    rng = np.random.default_rng(w.ids_seed)
    return rng.integers(0, w.model.vocab, size=(w.batch, w.prompt_len)).astype(np.int32)
