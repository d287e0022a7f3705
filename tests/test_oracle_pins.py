"""Pins of the CPU oracle to things other than itself (CPU only).

Each test names what fixes the expected value: a printed fact of the pages,
a library routine, a closed form, an invariant of the mathematics, or the
independent brute-force route of tests/bruteforce_ref.py.  The last group
plants plausible mistakes in the oracle and checks that a pin catches each.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import oracle.qwen2_oracle as OQ
import synthetic as S
from tests import bruteforce_ref as BF
from tests.helpers import with_random_norms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = S.WORKLOADS["tiny"]


def tiny_variant(**kw):
    return S.TINY.replace(**kw)


@pytest.fixture(scope="module")
def tiny_model():
    W = S.make_weights(TINY.model, 0)
    return W, O.OracleModel(TINY.model, W), S.make_ids(TINY)[0]


# ------------------------------------------------------------ printed facts
def test_param_count_matches_page():
    """The 1.5B shape bookkeeping (tied embedding, q/k/v bias only) reproduces
    the parameter count the 1.5B engine page prints."""
    facts = json.load(open(os.path.join(GOLDEN, "qwen25_1p5b_facts.json")))
    m = S.QWEN25_15B
    assert S.param_count(m) == facts["parameters"]
    assert (m.n_layers, m.n_heads, m.n_kv_heads) == (facts["layers"], facts["query_heads"], facts["kv_heads"])


def test_coder7b_config_shapes_consistent():
    """The 7B config printed in the speedrun listing: head_dim * heads = hidden,
    heads divisible by KV heads (GQA)."""
    c = json.load(open(os.path.join(GOLDEN, "qwen25_coder_7b_config.json")))
    assert c["num_heads"] * c["head_dim"] == c["hidden_size"]
    assert c["num_heads"] % c["num_kv_heads"] == 0
    m = S.ModelShape("coder-7b", c["num_layers"], c["hidden_size"], c["num_heads"], c["num_kv_heads"],
                     c["head_dim"], c["intermediate_size"], c["vocab_size"], tie_embeddings=False)
    # untied head: one more V x H matrix than the tied count
    assert S.param_count(m) - S.param_count(m.replace(tie_embeddings=True)) == c["vocab_size"] * c["hidden_size"]


# ------------------------------------------------------------ weight reading
def test_bf16_reading_is_exact_vs_torch():
    rng = np.random.default_rng(5)
    f = (rng.standard_normal(4096).astype(np.float32) * np.float32(0.02))
    f[:4] = [0.0, -0.0, 1e-30, 3.0e38]
    bits = S.f32_to_bf16_bits(f)
    via_torch = torch.from_numpy(f).bfloat16()                 # torch rounds to nearest even
    assert np.array_equal(bits.view(np.int16), via_torch.view(torch.int16).numpy())
    assert np.array_equal(O.decode_storage(bits), via_torch.double().numpy())


def test_f16_reading_is_exact_vs_torch():
    rng = np.random.default_rng(6)
    f = (rng.standard_normal(4096).astype(np.float32) * np.float32(0.02)).astype(np.float16)
    f[:3] = [0.0, 6.0e-8, 65504.0]                            # zero, smallest subnormal, largest normal
    assert np.array_equal(O.decode_storage(f), torch.from_numpy(f).double().numpy())


# ------------------------------------------------------------ RoPE
def test_rope_matches_complex_multiplication():
    """Split-half RoPE is multiplication of (x_i + i x_{i+hd/2}) by exp(i pos f_i)."""
    rng = np.random.default_rng(0)
    hd, theta = 64, 1e6
    x = rng.standard_normal((5, 3, hd))
    pos = np.array([0, 1, 7, 513, 8319])
    got = O.rope_rotate(x, pos, theta)
    z = x[..., :hd // 2] + 1j * x[..., hd // 2:]
    ang = pos[:, None, None] * (theta ** (-np.arange(hd // 2) * 2.0 / hd))[None, None, :]
    w = z * np.exp(1j * ang)
    np.testing.assert_allclose(got, np.concatenate([w.real, w.imag], -1), rtol=0, atol=1e-12)


def test_rope_matches_permuted_block_rotation():
    rng = np.random.default_rng(1)
    hd = 32
    x = rng.standard_normal((1, 1, hd))
    for pos in (0, 3, 17):
        R = BF.rotation_matrix(pos, hd, 1e6)
        np.testing.assert_allclose(O.rope_rotate(x, np.array([pos]), 1e6)[0, 0], R @ x[0, 0], atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    hd = 128
    q, k = rng.standard_normal((2, 1, 1, hd))
    # identity at position 0
    np.testing.assert_array_equal(O.rope_rotate(q, np.array([0]), 1e6), q)
    # norm preserved
    for p in (1, 100, 8319):
        r = O.rope_rotate(q, np.array([p]), 1e6)
        assert abs(np.linalg.norm(r) - np.linalg.norm(q)) < 1e-12 * np.linalg.norm(q)
    # q.k depends only on the position offset
    def dot(m, n):
        return float(np.sum(O.rope_rotate(q, np.array([m]), 1e6) * O.rope_rotate(k, np.array([n]), 1e6)))
    for m, n, s in ((5, 2, 11), (40, 40, 1000), (3, 9, 8000)):
        assert abs(dot(m, n) - dot(m + s, n + s)) < 1e-9


def test_rope_frequency_table_closed_form():
    f = O.rope_inverse_frequencies(8, 10000.0)
    np.testing.assert_allclose(f, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)


# ------------------------------------------------------------ attention
def test_softmax_rows_sum_to_one_and_mask_is_exact_zero():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((7, 16)), rng.standard_normal((10, 16))
    p = O.attention_weights(q, k, np.arange(3, 10), np.arange(10))
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)
    for t, qp in enumerate(range(3, 10)):
        assert np.all(p[t, qp + 1:] == 0.0) and np.all(p[t, :qp + 1] > 0)


def test_attention_matches_torch_sdpa_with_repeated_kv():
    rng = np.random.default_rng(4)
    T, nq, nkv, hd = 9, 6, 2, 16
    q = rng.standard_normal((T, nq, hd))
    k = rng.standard_normal((T, nkv, hd))
    v = rng.standard_normal((T, nkv, hd))
    got = O.causal_gqa_attention(q, k, v, np.arange(T), np.arange(T))
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(np.repeat(k, nq // nkv, axis=1)).permute(1, 0, 2).contiguous()
    tv = torch.from_numpy(np.repeat(v, nq // nkv, axis=1)).permute(1, 0, 2).contiguous()
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_single_key_attention_returns_value_exactly():
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((3, 1, 4, 32))
    q = np.concatenate([q] * 2, axis=1)     # 8 query heads over 4 KV heads
    out = O.causal_gqa_attention(q, k, v, np.array([0]), np.array([0]))
    for h in range(8):
        np.testing.assert_array_equal(out[0, h], v[0, h // 2])


def test_zero_query_gives_causal_running_mean():
    rng = np.random.default_rng(7)
    T = 6
    q = np.zeros((T, 2, 8))
    k, v = rng.standard_normal((2, T, 1, 8))
    out = O.causal_gqa_attention(q, k, v, np.arange(T), np.arange(T))
    for t in range(T):
        np.testing.assert_allclose(out[t, 0], v[:t + 1, 0].mean(0), atol=1e-14)


# ------------------------------------------------------------ small ops vs torch
def test_rms_norm_matches_torch():
    rng = np.random.default_rng(8)
    x, w = rng.standard_normal((5, 96)) * 3, rng.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-6), ref, atol=1e-13)


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), atol=1e-15)


def test_greedy_takes_lowest_index_on_ties():
    lg = np.array([0.5, 2.0, -1.0, 2.0, 2.0])
    assert O.greedy_token(lg) == 1 == int(torch.argmax(torch.from_numpy(lg)))


# ------------------------------------------------------------ whole-model pins
def _hf_model(m):
    from transformers import Qwen2Config, Qwen2ForCausalLM
    cfg = Qwen2Config(vocab_size=m.vocab, hidden_size=m.hidden, intermediate_size=m.intermediate,
                      num_hidden_layers=m.n_layers, num_attention_heads=m.n_heads,
                      num_key_value_heads=m.n_kv_heads, rms_norm_eps=m.rms_eps, rope_theta=m.rope_theta,
                      tie_word_embeddings=True, max_position_embeddings=256, attn_implementation="eager")
    torch.manual_seed(0)
    return Qwen2ForCausalLM(cfg).double().eval()


def _hf_logits(m, W, seq):
    hf = _hf_model(m)
    sd = {k: torch.from_numpy(O.decode_storage(v)) for k, v in W.items()}
    res = hf.load_state_dict(sd, strict=False)
    assert set(res.missing_keys) <= {"lm_head.weight"} and not res.unexpected_keys
    assert hf.lm_head.weight.data_ptr() == hf.model.embed_tokens.weight.data_ptr()    # tied
    with torch.no_grad():
        return hf(torch.tensor([list(seq)], dtype=torch.long)).logits[0].numpy()


# HF evaluates RoPE's cos/sin in float32 even in a float64 model (about 1e-7
# relative here); any of the planted mistakes below moves logits by > 1e-3.
HF_TOL = 2e-5


@pytest.mark.parametrize("shape,random_norms", [
    (S.TINY, False),
    (S.TINY, True),
    (S.TINY.replace(n_kv_heads=1), False),            # multi-query
    (S.TINY.replace(n_kv_heads=4), True),             # plain multi-head
    (S.TINY.replace(dtype="bf16", vocab=1000), True),
])
def test_oracle_matches_transformers_qwen2(shape, random_norms):
    W = S.make_weights(shape, 3)
    if random_norms:
        W = with_random_norms(W, shape)
    ids = np.random.default_rng(11).integers(0, shape.vocab, 13)
    om = O.OracleModel(shape, W)
    got = om.forward(ids, 0, om.new_cache(16), logits_rows=slice(0, 13))
    ref = _hf_logits(shape, W, ids)
    assert np.abs(got - ref).max() < HF_TOL


def test_cached_decode_matches_transformers_qwen2(tiny_model):
    W, om, ids = tiny_model
    toks, logits = om.generate(ids, TINY.decode_steps)
    ref = _hf_logits(TINY.model, W, list(ids) + list(toks[:-1]))[len(ids) - 1:]
    assert np.abs(logits - ref).max() < HF_TOL


def test_oracle_matches_bruteforce(tiny_model):
    W, om, ids = tiny_model
    toks, logits = om.generate(ids[:6], 3)
    bt, bl = BF.generate(TINY.model, W, ids[:6], 3)
    assert np.abs(logits - bl).max() < 1e-12
    assert np.array_equal(toks, bt)


@pytest.mark.parametrize("nkv", [1, 2, 4])
def test_oracle_matches_bruteforce_gqa_variants(nkv):
    m = S.TINY.replace(n_kv_heads=nkv, n_layers=1, vocab=300)
    W = S.make_weights(m, 9)
    ids = np.random.default_rng(nkv).integers(0, m.vocab, 5)
    om = O.OracleModel(m, W)
    got = om.forward(ids, 0, om.new_cache(5), logits_rows=slice(0, 5))
    assert np.abs(got - BF.full_forward(m, W, list(ids))).max() < 1e-12


def test_cached_equals_uncached(tiny_model):
    _, om, ids = tiny_model
    toks, logits = om.generate(ids, 8)
    tf = om.teacher_forced(ids, toks[:-1])
    assert np.abs(tf - logits).max() < 1e-12


def test_causal_invariance_bit_identical(tiny_model):
    _, om, ids = tiny_model
    a = om.forward(ids, 0, om.new_cache(16), logits_rows=slice(0, 16))
    ids2 = ids.copy()
    ids2[9:] = (ids2[9:] + 17) % TINY.model.vocab
    b = om.forward(ids2, 0, om.new_cache(16), logits_rows=slice(0, 16))
    assert np.array_equal(a[:9], b[:9])
    assert not np.array_equal(a[9:], b[9:])


def test_gqa_equals_mha_with_repeated_kv_weights():
    m = S.TINY.replace(vocab=500)
    W = S.make_weights(m, 4)
    g = m.group
    mha = m.replace(n_kv_heads=m.n_heads)
    W2 = dict(W)
    for l in range(m.n_layers):
        for t in ("k", "v"):
            wk = W[f"model.layers.{l}.self_attn.{t}_proj.weight"].reshape(m.n_kv_heads, m.head_dim, m.hidden)
            bk = W[f"model.layers.{l}.self_attn.{t}_proj.bias"].reshape(m.n_kv_heads, m.head_dim)
            W2[f"model.layers.{l}.self_attn.{t}_proj.weight"] = np.repeat(wk, g, 0).reshape(-1, m.hidden)
            W2[f"model.layers.{l}.self_attn.{t}_proj.bias"] = np.repeat(bk, g, 0).reshape(-1)
    ids = S.make_ids(TINY)[0] % m.vocab
    a = O.OracleModel(m, W).generate(ids, 4)[1]
    b = O.OracleModel(mha, W2).generate(ids, 4)[1]
    assert np.abs(a - b).max() < 1e-12


def test_first_layer_closed_form_single_token():
    """One token at position 0: RoPE is the identity, attention returns v, so
    layer 0 is a closed form of the embedding row."""
    m = S.TINY.replace(n_layers=1)
    W = S.make_weights(m, 2)
    D = {k: O.decode_storage(v) for k, v in W.items()}
    tok = 77
    x = D["model.embed_tokens.weight"][tok]
    p = "model.layers.0."
    u = x / math.sqrt(np.mean(x * x) + 1e-6)
    v = D[p + "self_attn.v_proj.weight"] @ u + D[p + "self_attn.v_proj.bias"]
    o = np.concatenate([v[(h // m.group) * m.head_dim:(h // m.group + 1) * m.head_dim] for h in range(m.n_heads)])
    x1 = x + D[p + "self_attn.o_proj.weight"] @ o
    u2 = x1 / math.sqrt(np.mean(x1 * x1) + 1e-6)
    gt = D[p + "mlp.gate_proj.weight"] @ u2
    x2 = x1 + D[p + "mlp.down_proj.weight"] @ (gt / (1 + np.exp(-gt)) * (D[p + "mlp.up_proj.weight"] @ u2))
    y = x2 / math.sqrt(np.mean(x2 * x2) + 1e-6)
    om = O.OracleModel(m, W)
    np.testing.assert_allclose(om.forward([tok], 0, om.new_cache(1)), D["model.embed_tokens.weight"] @ y, atol=1e-12)


# ------------------------------------------------------------ planted mistakes
_ROPE = OQ.rope_rotate
_ATTW = OQ.attention_weights


def _rope_wrong_sign(x, positions, theta):
    return _ROPE(x, -np.asarray(positions), theta)


def _rope_interleaved(x, positions, theta):
    hd = x.shape[-1]
    perm = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])
    inv = np.argsort(perm)
    return _ROPE(x[..., perm], positions, theta)[..., inv]


def _gqa_modulo(q, k, v, q_pos, k_pos):
    nkv = k.shape[1]
    out = np.empty(q.shape)
    for h in range(q.shape[1]):
        out[:, h] = _ATTW(q[:, h], k[:, h % nkv], q_pos, k_pos) @ v[:, h % nkv]
    return out


def _rms_without_weight(x, w, eps):
    return x / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps)


def _rms_sum_not_mean(x, w, eps):
    return x / np.sqrt(np.sum(x * x, -1, keepdims=True) + eps) * w


def _attn_no_scale(q, k, q_pos, k_pos):
    return _ATTW(q * math.sqrt(q.shape[-1]), k, q_pos, k_pos)


@pytest.mark.parametrize("name,fake", [
    ("rope_rotate", _rope_wrong_sign),
    ("rope_rotate", _rope_interleaved),
    ("causal_gqa_attention", _gqa_modulo),
    ("rms_norm", _rms_without_weight),
    ("rms_norm", _rms_sum_not_mean),
    ("attention_weights", _attn_no_scale),
])
def test_pins_catch_planted_mistakes(monkeypatch, name, fake):
    monkeypatch.setattr(OQ, name, fake)
    m = S.TINY
    W = with_random_norms(S.make_weights(m, 3), m)
    ids = np.random.default_rng(11).integers(0, m.vocab, 13)
    om = O.OracleModel(m, W)
    got = om.forward(ids, 0, om.new_cache(16), logits_rows=slice(0, 13))
    assert np.abs(got - _hf_logits(m, W, ids)).max() > 100 * HF_TOL


# ------------------------------------------------------------ sampling
def test_philox_matches_numpy():
    """The oracle's Philox-4x64-10 against numpy's bit generator of the same
    name (numpy's first block uses counter + 1)."""
    for key, ctr in (([5, 7], [0, 0, 0, 0]), ([2 ** 64 - 1, 3], [41, 9, 0, 2 ** 63])):
        g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
        want = [int(x) for x in g.random_raw(4)]
        c1 = list(ctr)
        c1[0] = (c1[0] + 1) % 2 ** 64
        assert O.philox4x64_10(c1, key) == want


def test_sampling_draw_range():
    us = [O.sampling_draw(3, b, n) for b in range(4) for n in range(200)]
    assert all(0.0 <= u < 1.0 for u in us)
    assert abs(np.mean(us) - 0.5) < 0.05 and len(set(us)) == len(us)


def test_sample_token_special_cases():
    rng = np.random.default_rng(9)
    lg = rng.standard_normal(50)
    am = int(np.argmax(lg))
    for u in (0.0, 0.3, 0.999):
        assert O.sample_token(lg, 1.0, 1, 1.0, u)[0] == am          # top_k = 1 is greedy
        assert O.sample_token(lg, 1e-4, 50, 1.0, u)[0] == am         # a cold temperature too
        assert O.sample_token(lg, 0.7, 50, 1e-9, u)[0] == am         # top_p -> 0 keeps one token
    tie = np.array([0.0, 2.0, 2.0, 1.0])
    assert O.sample_token(tie, 1.0, 1, 1.0, 0.5)[0] == 1             # equal maxima: lower index


def test_sample_token_is_the_inverse_cdf_of_the_filtered_softmax():
    """Brute force: a fine grid of draws u maps to each kept token with the
    frequency of its renormalised probability, and top-p keeps the shortest
    prefix reaching top_p."""
    lg = np.log(np.array([0.1, 0.5, 0.05, 0.3, 0.05]))
    # top_k = 4 drops one 0.05 (index 4, the higher index of the tie)
    _, order, C, m, _ = O.sample_token(lg, 1.0, 4, 1.0, 0.0)
    assert list(order) == [1, 3, 0, 2] and m == 4
    # top_p = 0.8 of the top-4 mass 0.95 is 0.76: prefix sums 0.5, 0.8, ... reach it at the second
    _, _, C, m, _ = O.sample_token(lg, 1.0, 4, 0.8, 0.0)
    assert m == 2
    grid = (np.arange(100000) + 0.5) / 100000
    toks = np.array([O.sample_token(lg, 1.0, 4, 0.8, u)[0] for u in grid])
    assert set(toks) == {1, 3}
    assert abs((toks == 1).mean() - 0.5 / 0.8) < 1e-4
    # temperature 2 flattens: weights p ** (1 / 2)
    p2 = np.sqrt(np.array([0.1, 0.5, 0.05, 0.3, 0.05]))
    toks = np.array([O.sample_token(lg, 2.0, 5, 1.0, u)[0] for u in grid[::10]])
    for i in range(5):
        assert abs((toks == i).mean() - p2[i] / p2.sum()) < 2e-4
