"""Parity of the HIP library (through its C ABI) with the CPU oracle.

Every case runs prefill + greedy decode on the GPU, then feeds the GPU's own
token stream to the oracle (teacher forcing) and compares logits at every
step and tokens wherever the oracle's top-2 margin is clear.
"""
import sys

import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests.helpers import LOGIT_TOL, assert_same_sequence, compare_row, gpu_generate, with_random_norms

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def Q():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_only_transformer_qwen2_amd as Q
    Q.load_library()
    return Q


def make(Q, shape, W, max_batch, max_seq):
    return Q.Model(shape, Q.device_tensors(shape, W), max_batch, max_seq)


SMALL = {
    # several 64-wide tiles with ragged tails (vocab, prompt, intermediate)
    "bf16-hd32": (S.ModelShape("s32", 3, 256, 8, 2, 32, 640, 1000), 3, 37, 6, 64),
    "bf16-hd64-mqa": (S.ModelShape("s64", 2, 384, 6, 1, 64, 1024, 777), 2, 70, 5, 96),
    "bf16-hd128": (S.ModelShape("s128", 2, 512, 4, 2, 128, 1536, 2049), 2, 130, 4, 160),
    "f32-hd64": (S.ModelShape("f64", 2, 192, 6, 3, 64, 448, 513, dtype="f32"), 2, 21, 5, 32),
    # fp16 weights (the same kernels; the caller's fp16 tensors are scaled like bf16 ones)
    "f16-hd128": (S.ModelShape("h128", 2, 512, 4, 2, 128, 1536, 2049, dtype="f16"), 2, 130, 4, 160),
    "f16-hd64-g7-b5": (S.ModelShape("h64g7", 2, 448, 14, 2, 64, 896, 1100, dtype="f16"), 5, 53, 6, 96),
    # more than two rows: the batched decode path (split-KV attention on the
    # matrix cores, g = 7 as in the 0.5B model; unsplit gate/up with SwiGLU)
    "bf16-hd64-g7-b5": (S.ModelShape("s64g7", 2, 448, 14, 2, 64, 896, 1100), 5, 53, 6, 96),
    # 17..32 rows: two 16-row MFMA column blocks in the batched projections
    # (K split with atomics for q/k/v, o and down; g = 6 as in the 1.5B model)
    "bf16-hd64-g6-b20": (S.ModelShape("s64g6", 2, 512, 12, 2, 64, 1088, 1500), 20, 33, 5, 64),
    # eight query heads per KV head (the widest group the decode attention
    # takes), one row and a batch
    "bf16-hd64-g8-b1": (S.ModelShape("s64g8", 2, 512, 8, 1, 64, 1024, 1500), 1, 45, 5, 64),
    "bf16-hd64-g8-b5": (S.ModelShape("s64g8", 2, 512, 8, 1, 64, 1024, 1500), 5, 45, 5, 64),
    # plain multi-head attention (one query head per KV head)
    "bf16-hd64-mha-b1": (S.ModelShape("s64mha", 2, 256, 4, 4, 64, 512, 999), 1, 30, 5, 48),
    "bf16-hd64-mha-b3": (S.ModelShape("s64mha", 2, 256, 4, 4, 64, 512, 999), 3, 30, 5, 48),
    # the 1.5B model's widths (hidden 1536, 12/2 heads of 128, intermediate
    # 8960) in two layers: the decode kernels instantiated for them (norm
    # prologues over K = 1536, the one-row MLP with late down-projection
    # loads, the wide merged attention + o projection) under random norm
    # weights; one row crosses the 256-key switch to the split-KV pair
    "bf16-h1536-b1": (S.ModelShape("s1536", 2, 1536, 12, 2, 128, 8960, 3001), 1, 250, 10, 272),
    "bf16-h1536-b2": (S.ModelShape("s1536", 2, 1536, 12, 2, 128, 8960, 3001), 2, 61, 5, 72),
    # the Coder-7B widths (hidden 3584, 28/4 heads of 128, intermediate 18944,
    # untied LM head) in two layers: one row across the 256-key switch (norm
    # prologues over K = 3584, the MLP as two projections since hidden exceeds
    # the one-kernel MLP), and five rows (batched projections, g = 7 at head
    # dim 128)
    "bf16-h3584-g7-b1": (S.ModelShape("s3584", 2, 3584, 28, 4, 128, 18944, 5003, tie_embeddings=False),
                         1, 250, 10, 272),
    "bf16-h3584-g7-b5": (S.ModelShape("s3584", 2, 3584, 28, 4, 128, 18944, 5003, tie_embeddings=False),
                         5, 40, 5, 64),
}


@pytest.mark.parametrize("graph", [True, False])
def test_tiny_fp32_full_workload(Q, graph):
    w = S.WORKLOADS["tiny"]
    W = with_random_norms(S.make_weights(w.model, 0), w.model)
    ids = S.make_ids(w)
    say(f"tiny fp32 B={w.batch} P={w.prompt_len} D={w.decode_steps} graph={graph}")
    m = make(Q, w.model, W, w.batch, w.max_seq)
    toks, logits = gpu_generate(m, ids, w.decode_steps, graph=graph)
    om = O.OracleModel(w.model, W)
    err, n = compare_row(om, ids[0], toks[0], logits[0], "f32", "tiny")
    say(f"  max err {err:.2e}, {n} steps with a clear margin")
    # free-running agreement with the oracle's own generation
    o_toks, _ = om.generate(ids[0], w.decode_steps)
    say(f"  oracle tokens {o_toks}, gpu tokens {toks[0]}")


@pytest.mark.parametrize("case", list(SMALL))
def test_small_shapes(Q, case):
    shape, B, P, D, smax = SMALL[case]
    W = with_random_norms(S.make_weights(shape, 5), shape)
    ids = np.random.default_rng(7).integers(0, shape.vocab, (B, P)).astype(np.int32)
    say(f"{case}: B={B} P={P} D={D}")
    m = make(Q, shape, W, B, smax)
    toks, logits = gpu_generate(m, ids, D)
    om = O.OracleModel(shape, W)
    for b in range(B):
        err, n = compare_row(om, ids[b], toks[b], logits[b], shape.dtype, f"{case} row {b}")
        say(f"  row {b}: max err {err:.2e}")


def test_graph_and_eager_bit_identical(Q):
    shape, B, P, D, smax = SMALL["bf16-hd64-mqa"]
    W = S.make_weights(shape, 1)
    ids = np.random.default_rng(3).integers(0, shape.vocab, (B, P)).astype(np.int32)
    m = make(Q, shape, W, B, smax)
    t1, l1 = gpu_generate(m, ids, D, graph=True)
    t2, l2 = gpu_generate(m, ids, D, graph=False)
    assert np.array_equal(t1, t2) and np.array_equal(l1, l2)


def test_logits_all_and_causal_invariance(Q):
    import torch
    shape, B, P, D, smax = SMALL["bf16-hd32"]
    W = S.make_weights(shape, 2)
    ids = np.random.default_rng(4).integers(0, shape.vocab, (B, P)).astype(np.int32)
    m = make(Q, shape, W, B, smax)

    def all_logits(ids_np):
        t = torch.from_numpy(ids_np).cuda()
        lg = torch.empty((B, P, shape.vocab), dtype=torch.float32, device="cuda")
        nxt = m.prefill(t, logits=lg, logits_all=True)
        torch.cuda.synchronize()
        return lg.cpu().numpy(), nxt.cpu().numpy()

    a, na = all_logits(ids)
    om = O.OracleModel(shape, W)
    for b in range(B):
        ref = om.forward(ids[b], 0, om.new_cache(P), logits_rows=slice(0, P))
        assert np.abs(a[b] - ref).max() <= LOGIT_TOL["bf16"]
        assert na[b] == int(np.argmax(a[b, -1]))
    ids2 = ids.copy()
    ids2[:, 20:] = (ids2[:, 20:] + 1) % shape.vocab
    c, _ = all_logits(ids2)
    assert np.array_equal(a[:, :20], c[:, :20])        # rows before the change: bit-identical
    assert not np.array_equal(a[:, 20:], c[:, 20:])


def test_cached_decode_equals_full_prefill(Q):
    """Decode-step logits equal the logits_all of one prefill over the prompt
    plus the emitted tokens (same kernels, different row counts)."""
    import torch
    shape, B, P, D, smax = SMALL["bf16-hd128"]
    W = S.make_weights(shape, 3)
    ids = np.random.default_rng(5).integers(0, shape.vocab, (B, P)).astype(np.int32)
    m = make(Q, shape, W, B, smax)
    toks, logits = gpu_generate(m, ids, D)
    full = np.concatenate([ids, toks[:, :-1]], axis=1).astype(np.int32)
    lg = torch.empty((B, P + D, shape.vocab), dtype=torch.float32, device="cuda")
    m.prefill(torch.from_numpy(full).cuda(), logits=lg, logits_all=True)
    torch.cuda.synchronize()
    ref = lg.cpu().numpy()[:, P - 1:]
    assert np.abs(ref - logits).max() <= LOGIT_TOL["bf16"] / 10


def test_batch_rows_are_independent(Q):
    shape, B, P, D, smax = SMALL["bf16-hd32"]
    W = S.make_weights(shape, 4)
    ids = np.random.default_rng(6).integers(0, shape.vocab, (B, P)).astype(np.int32)
    m = make(Q, shape, W, B, smax)
    tb, lb = gpu_generate(m, ids, D)
    for b in range(B):
        t1, l1 = gpu_generate(m, ids[b:b + 1], D)
        assert_same_sequence(tb[b], lb[b], t1[0], l1[0], label=f"row {b} vs batch-1")


def test_prompt_of_one_and_full_cache(Q):
    import torch
    shape = SMALL["bf16-hd64-mqa"][0]
    W = S.make_weights(shape, 8)
    smax = 12
    m = make(Q, shape, W, 2, smax)
    om = O.OracleModel(shape, W)
    ids = np.array([[5], [700]], dtype=np.int32)
    toks, logits = gpu_generate(m, ids, smax - 1)            # positions 0 .. smax-1: cache exactly full
    for b in range(2):
        compare_row(om, ids[b], toks[b], logits[b], "bf16", f"P=1 row {b}")
    assert m.state() == (2, smax)
    nxt = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(Q.QwError) as e:
        m.decode_step(torch.from_numpy(toks[:, -1].copy()).cuda(), next_ids=nxt)
    assert e.value.status == -4                              # QW_ERR_CACHE_FULL
    assert m.state() == (2, smax)


def test_error_paths(Q):
    import torch
    shape, B, P, D, smax = SMALL["bf16-hd32"]
    m = make(Q, shape, S.make_weights(shape, 0), 2, 16)
    ids = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    nxt = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(Q.QwError) as e:
        m.decode_step(ids[:, 0].contiguous(), next_ids=nxt)
    assert e.value.status == -5                              # BAD_STATE: no prefill yet
    with pytest.raises(Q.QwError) as e:
        m.prefill(torch.zeros((3, 4), dtype=torch.int32, device="cuda"))
    assert e.value.status == -1                              # batch > max_batch
    with pytest.raises(Q.QwError) as e:
        m.prefill(torch.zeros((1, 17), dtype=torch.int32, device="cuda"))
    assert e.value.status == -4                              # prompt longer than the cache
    bad = torch.tensor([[1, 2, shape.vocab, 3], [0, -1, 2, 3]], dtype=torch.int32, device="cuda")
    m.prefill(bad, next_ids=nxt)
    with pytest.raises(Q.QwError):
        m.check_ids()
    m.check_ids()                                            # flag was cleared
    with pytest.raises(Q.QwError):
        m.timing_enable("no_such_kernel")


@pytest.mark.parametrize("name", ["0.5b", "1.5b", "0.5b-f16"])
def test_full_workload(Q, name):
    """The workload at full size against the oracle, with norm weights drawn
    around 1 (the workloads' own norms are exactly 1); "0.5b-f16" is the 0.5B
    workload with fp16 weights."""
    w = S.WORKLOADS[name.replace("-f16", "")]
    if name.endswith("-f16"):
        w = w.replace(model=w.model.replace(dtype="f16"))
    say(f"{name}: generating weights")
    W = with_random_norms(S.make_weights(w.model, w.weight_seed), w.model)
    ids = S.make_ids(w)
    say(f"{name}: GPU B={w.batch} P={w.prompt_len} D={w.decode_steps}")
    m = make(Q, w.model, W, w.batch, w.max_seq)
    toks, logits = gpu_generate(m, ids, w.decode_steps)
    m.close()
    say(f"{name}: oracle teacher-forced")
    om = O.OracleModel(w.model, W)
    err, n = compare_row(om, ids[0], toks[0], logits[0], w.model.dtype, name)
    say(f"{name}: max err {err:.3e} over {w.decode_steps + 1} steps; {n} with margin > 0.1")


def test_full_workload_coder7b(Q):
    """The second model family: Qwen2.5-Coder-7B shapes with an untied LM head
    (28 layers, 15 GB of bf16 weights), one sequence of 512 prompt tokens and
    128 decode steps, against the oracle at every step, norm weights drawn
    around 1."""
    w = S.WORKLOADS["coder-7b"]
    say("coder-7b: generating weights")
    W = with_random_norms(S.make_weights(w.model, w.weight_seed), w.model)
    ids = S.make_ids(w)
    say(f"coder-7b: GPU B={w.batch} P={w.prompt_len} D={w.decode_steps}")
    m = make(Q, w.model, W, w.batch, w.max_seq)
    toks, logits = gpu_generate(m, ids, w.decode_steps)
    m.check_numerics()
    m.close()
    say("coder-7b: oracle teacher-forced")
    om = O.OracleModel(w.model, W)
    err, n = compare_row(om, ids[0], toks[0], logits[0], "bf16", "coder-7b")
    say(f"coder-7b: max err {err:.3e} over {w.decode_steps + 1} steps; {n} with margin > 0.1")


LONG = {
    # many 128-row query tiles and 64-key blocks, ragged ends
    "long-hd64": (S.ModelShape("l64", 2, 256, 6, 2, 64, 512, 1001), 2, 700, 3, 704),
    "long-hd128-8k": (S.ModelShape("l128", 2, 256, 6, 1, 128, 512, 999), 1, 8190, 4, 8194),
    # the 1.5B attention geometry (12 q heads over 2 KV heads, hd 128) at 8k
    "long-1.5b-attn-8k": (S.ModelShape("l15", 2, 512, 12, 2, 128, 512, 999), 1, 8192, 6, 8320),
    # two rows decoding across a context of 256 keys: the merged attention +
    # o projection kernel runs up to there, the split-KV pair after it (the
    # decode graph is captured again at the switch)
    "cross-256-hd64": (S.ModelShape("c64", 2, 256, 6, 2, 64, 512, 1003), 2, 252, 8, 300),
    # enough prompt rows that the q/k/v projection runs unsplit at head dims
    # 64 and 32 (bias + RoPE then in their own kernel; shorter prompts take
    # them in the projection's split-K reduction)
    "unsplit-qkv-hd64": (S.ModelShape("f64q", 2, 256, 8, 2, 64, 512, 997), 2, 1408, 3, 1412),
    "unsplit-qkv-hd32": (S.ModelShape("f32q", 2, 256, 8, 2, 32, 512, 995), 4, 1400, 3, 1404),
}


@pytest.mark.parametrize("case", list(LONG))
def test_long_prompts_small_model(Q, case):
    shape, B, P, D, smax = LONG[case]
    W = with_random_norms(S.make_weights(shape, 6), shape)
    ids = np.random.default_rng(8).integers(0, shape.vocab, (B, P)).astype(np.int32)
    say(f"{case}: B={B} P={P} D={D}")
    m = make(Q, shape, W, B, smax)
    toks, logits = gpu_generate(m, ids, D)
    om = O.OracleModel(shape, W)
    for b in range(B):
        err, n = compare_row(om, ids[b], toks[b], logits[b], shape.dtype, f"{case} row {b}")
        say(f"  row {b}: max err {err:.2e}")


def test_big_tile_epilogues(Q):
    """64 prompts of 2048 tokens on a small model: every prefill projection
    (q/k/v, o, gate/up, down) runs unsplit on 256 x 256 tiles, whose fp32
    store, residual-add and SwiGLU outputs go through LDS; rows 0 and 63 are
    checked against the oracle, the batch's first decode steps included."""
    shape = S.ModelShape("big", 2, 256, 4, 2, 64, 512, 1000)
    B, P, D = 64, 2048, 2
    T = B * P
    for N in (shape.q_dim + 2 * shape.kv_dim, shape.hidden, 2 * shape.intermediate):
        assert ((T + 255) // 256) * ((N + 255) // 256) >= 512       # the unsplit 256 x 256 kernel
    W = with_random_norms(S.make_weights(shape, 31), shape)
    ids = np.random.default_rng(32).integers(0, shape.vocab, (B, P)).astype(np.int32)
    m = make(Q, shape, W, B, P + D + 2)
    toks, logits = gpu_generate(m, ids, D)
    m.close()
    om = O.OracleModel(shape, W)
    for b in (0, B - 1):
        err, n = compare_row(om, ids[b], toks[b], logits[b], shape.dtype, f"big-tile row {b}")
        say(f"  big-tile row {b}: max err {err:.2e}")


def test_full_workload_prefill_heavy(Q):
    """Batch 8 x 2048 prompt tokens + 32 decode steps at Qwen2.5-1.5B shapes.
    The oracle checks rows 0 and 7 (about 6.5 TFLOP each in float64); row 7
    is also checked against a batch-1 run of the same prompt on the GPU."""
    w = S.WORKLOADS["1.5b-prefill"]
    say("1.5b-prefill: generating weights")
    W = S.make_weights(w.model, w.weight_seed)
    ids = S.make_ids(w)
    m = make(Q, w.model, W, w.batch, w.max_seq)
    say("1.5b-prefill: GPU batch run")
    toks, logits = gpu_generate(m, ids, w.decode_steps)
    t7, l7 = gpu_generate(m, ids[7:8], w.decode_steps)
    # the prefill GEMMs may split K differently at batch 8 and batch 1 (more
    # tiles, another split), so the two runs agree to rounding, not bit for bit
    d0 = float(np.abs(l7[0, 0] - logits[7, 0]).max())
    assert d0 <= 2e-2, f"row 7 prefill logits: batch 8 vs batch 1 differ by {d0:.3e}"
    d = assert_same_sequence(toks[7], logits[7], t7[0], l7[0], label="row 7 vs batch-1")
    say(f"1.5b-prefill: row 7 batch-8 vs batch-1 max diff {d:.2e}")
    m.close()
    om = O.OracleModel(w.model, W)
    for b in (0, 7):
        say(f"1.5b-prefill: oracle row {b}")
        err, n = compare_row(om, ids[b], toks[b], logits[b], "bf16", f"1.5b-prefill row {b}")
        say(f"1.5b-prefill: row {b} max err {err:.3e}; {n} steps with margin > 0.1")


@pytest.fixture(scope="module")
def longctx(Q):
    """Batch 32 x 8192 prompt tokens + 128 decode steps at Qwen2.5-1.5B shapes,
    run once on the GPU for the tests below: the batch run (rows 0 and 31
    kept), a batch-1 run of row 31, and the logits of one prefill over row 0's
    prompt + emitted tokens."""
    import torch
    w = S.WORKLOADS["1.5b-longctx"]
    say("1.5b-longctx: generating weights")
    W = S.make_weights(w.model, w.weight_seed)
    ids = S.make_ids(w)
    m = make(Q, w.model, W, w.batch, w.max_seq)
    say("1.5b-longctx: GPU batch run")
    toks, logits = gpu_generate(m, ids, w.decode_steps)
    m.check_numerics()
    keep = {b: (toks[b].copy(), logits[b].copy()) for b in (0, 31)}
    finite = bool(np.all(np.isfinite(logits)))
    del logits
    say("1.5b-longctx: batch-1 run of row 31")
    t31, l31 = gpu_generate(m, ids[31:32], w.decode_steps)
    say("1.5b-longctx: prefill over prompt + emitted tokens of row 0")
    seq = np.concatenate([ids[0], keep[0][0][:-1]]).astype(np.int32)[None]
    lg = torch.empty((1, seq.shape[1], w.model.vocab), dtype=torch.float32, device="cuda")
    m.prefill(torch.from_numpy(seq).cuda(), logits=lg, logits_all=True)
    torch.cuda.synchronize()
    uncached = lg[0, w.prompt_len - 1:].cpu().numpy()
    del lg
    m.close()
    torch.cuda.empty_cache()
    return {"w": w, "W": W, "ids": ids, "rows": keep, "finite": finite, "b1_31": (t31[0], l31[0]),
            "uncached0": uncached}


@pytest.fixture(scope="module")
def longctx_oracle(longctx):
    return O.OracleModel(longctx["w"].model, longctx["W"])


def test_longctx_rows_independent(longctx):
    assert longctx["finite"]
    t, l = longctx["rows"][31]
    d = assert_same_sequence(t, l, *longctx["b1_31"], label="row 31 vs batch-1")
    say(f"1.5b-longctx: row 31 batch-32 vs batch-1 max diff {d:.2e}")


@pytest.mark.parametrize("row", [0, 31])
def test_longctx_oracle(longctx, longctx_oracle, row):
    t, l = longctx["rows"][row]
    say(f"1.5b-longctx: oracle row {row} (teacher-forced over {longctx['w'].prompt_len + len(t) - 1} positions)")
    ref = longctx_oracle.teacher_forced(longctx["ids"][row], t[:-1],
                                        progress=lambda l: l % 4 == 3 and say(f"  oracle layer {l + 1} done"))
    err, n = compare_row(longctx_oracle, longctx["ids"][row], t, l, "bf16", f"1.5b-longctx row {row}", ref=ref)
    say(f"1.5b-longctx: row {row} max err {err:.3e}; {n} steps with margin > 0.1")
    if row == 0:
        e_un = float(np.abs(longctx["uncached0"] - ref).max())
        say(f"1.5b-longctx: row 0 uncached (prefill logits) vs oracle {e_un:.3e}")
        assert e_un <= LOGIT_TOL["bf16"]


def test_longctx_cached_equals_uncached(longctx):
    """Decode logits of row 0 against the logits of one prefill over prompt +
    emitted tokens (P5 at full size).  Both are f16-operand approximations of
    the same forward that round and sum in different orders; each is checked
    against the oracle in test_longctx_oracle, where both measured about
    8.4e-3 from it at this workload.  Their distance is held to a third of
    the oracle tolerance, twice that measured drift."""
    diff = float(np.abs(longctx["uncached0"] - longctx["rows"][0][1]).max())
    say(f"1.5b-longctx: cached vs uncached max diff {diff:.3e}")
    assert diff <= LOGIT_TOL["bf16"] / 3
