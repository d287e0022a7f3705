"""The seeded input generator: deterministic, shaped as the HF checkpoints,
drawn as stated in its header (CPU only)."""
import numpy as np

import synthetic as S


def test_weights_are_deterministic_and_subsettable():
    m = S.TINY.replace(dtype="bf16")
    a = S.make_weights(m, 0)
    b = S.make_weights(m, 0, only={"model.layers.1.mlp.up_proj.weight"})
    assert np.array_equal(a["model.layers.1.mlp.up_proj.weight"], b["model.layers.1.mlp.up_proj.weight"])
    c = S.make_weights(m, 1)
    assert not np.array_equal(a["model.embed_tokens.weight"], c["model.embed_tokens.weight"])


def test_shapes_dtypes_and_init():
    for m in (S.TINY, S.TINY.replace(dtype="bf16")):
        W = S.make_weights(m, 0)
        assert list(W) == S.tensor_names(m)
        for k, v in W.items():
            assert v.shape == S.tensor_shape(m, k)
            assert v.dtype == (np.uint16 if m.dtype == "bf16" else np.float32)
        f = W["model.layers.0.mlp.gate_proj.weight"]
        if m.dtype == "bf16":
            f = (f.astype(np.uint32) << 16).view(np.float32)
        assert abs(float(f.std()) - 0.02) < 0.002 and abs(float(f.mean())) < 0.002
        n = W["model.layers.0.input_layernorm.weight"]
        assert np.all(n == (0x3F80 if m.dtype == "bf16" else 1.0))


def test_ids_uniform_in_vocab():
    w = S.WORKLOADS["0.5b"]
    ids = S.make_ids(w)
    assert ids.shape == (1, 128) and ids.dtype == np.int32
    assert ids.min() >= 0 and ids.max() < w.model.vocab
    assert np.array_equal(ids, S.make_ids(w))


def test_workload_table():
    W = S.WORKLOADS
    five = ["tiny", "0.5b", "1.5b", "1.5b-prefill", "1.5b-longctx"]
    assert [W[k].batch for k in five] == [1, 1, 1, 8, 32]
    assert [W[k].prompt_len for k in five] == [16, 128, 512, 2048, 8192]
    assert [W[k].decode_steps for k in five] == [8, 128, 256, 32, 128]
    assert set(W) == set(five) | {"coder-7b"}
    for w in W.values():
        assert w.prompt_len + w.decode_steps <= w.max_seq


def test_coder7b_shape_matches_the_listed_config():
    """The 7B workload's shape is the config the speedrun page prints
    (tests/golden/qwen25_coder_7b_config.json), with an untied LM head."""
    import json
    import os
    c = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "qwen25_coder_7b_config.json")))
    m = S.WORKLOADS["coder-7b"].model
    assert (m.n_layers, m.hidden, m.n_heads, m.n_kv_heads, m.head_dim, m.intermediate, m.vocab) == (
        c["num_layers"], c["hidden_size"], c["num_heads"], c["num_kv_heads"], c["head_dim"],
        c["intermediate_size"], c["vocab_size"])
    assert m.rope_theta == c["rope_theta"] and m.rms_eps == c["rms_norm_eps"]
    assert not m.tie_embeddings and "lm_head.weight" in S.tensor_names(m)


def test_ragged_workload_lengths():
    """The ragged serving batch: 32 seeded lengths within [256, 8192], the
    prompts of those lengths with ids in range, the same on every call."""
    w = S.RAGGED_WORKLOADS["1.5b-ragged"]
    lens = w.lengths()
    assert len(lens) == 32 and min(lens) >= 256 and max(lens) <= 8192
    assert lens == w.lengths() and len(set(lens)) > 16
    ps = w.prompts()
    assert [len(p) for p in ps] == lens
    assert all(p.dtype == np.int32 and p.min() >= 0 and p.max() < w.model.vocab for p in ps)
