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
    assert [W[k].batch for k in W] == [1, 1, 1, 8, 32]
    assert [W[k].prompt_len for k in W] == [16, 128, 512, 2048, 8192]
    assert [W[k].decode_steps for k in W] == [8, 128, 256, 32, 128]
    for w in W.values():
        assert w.prompt_len + w.decode_steps <= w.max_seq
