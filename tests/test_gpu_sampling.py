"""Sampling (temperature, top-k, top-p with a counter-based draw) and the
end-of-sequence rule on the device ("augur": sampling and EOS stopping; the
speedrun harness stops on the end-of-stream token)."""
import sys

import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests.helpers import LOGIT_TOL, gpu_generate

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


SHAPE = S.ModelShape("smp", 2, 448, 14, 2, 64, 896, 1100)


def check_choice(logits, tok, temperature, top_k, top_p, u, label):
    """The oracle's sampler on the same logits: the same token, or, when the
    draw falls within 1e-4 of the kept total from a cumulative-weight boundary
    (fp32 on the device, fp64 here), a neighbour of that boundary."""
    want, order, C, m, r = O.sample_token(logits, temperature, top_k, top_p, u)
    if tok == want:
        return True
    pos = np.nonzero(order[:m] == tok)[0]
    assert pos.size, f"{label}: token {tok} is not among the kept candidates {order[:m]}"
    j = int(pos[0])
    lo = C[j - 1] if j > 0 else 0.0
    near = min(abs(r - lo), abs(r - C[j])) <= 1e-4 * C[m - 1] or abs(top_p * C[-1] - C[m - 1]) <= 1e-4 * C[-1]
    assert near, f"{label}: token {tok} (rank {j}) for r = {r:.6g}, oracle {want}; C = {C[:m]}"
    return False


@pytest.mark.parametrize("B,graph", [(1, True), (3, True), (3, False)])
def test_sampled_tokens_follow_the_oracle_sampler(Q, B, graph):
    """Every step's token is the oracle sampler's choice on the step's own
    logits with the same draw; the logits match the oracle's forward over the
    sampled stream."""
    W = S.make_weights(SHAPE, 51)
    P, D = 24, 10
    ids = np.random.default_rng(52).integers(0, SHAPE.vocab, (B, P)).astype(np.int32)
    m = Q.Model(SHAPE, Q.device_tensors(SHAPE, W), B, P + D + 2)
    temp, k, p, seed = 0.8, 50, 0.9, 123
    m.set_sampling(temp, k, p, seed)
    toks, logits = gpu_generate(m, ids, D, graph=graph)
    m.close()
    om = O.OracleModel(SHAPE, W)
    exact = 0
    for b in range(B):
        for s_ in range(D + 1):
            u = O.sampling_draw(seed, b, P + s_)
            exact += check_choice(logits[b, s_], int(toks[b, s_]), temp, k, p, u, f"row {b} step {s_}")
        ref = om.teacher_forced(ids[b], toks[b, :-1])
        err = np.abs(logits[b] - ref).max()
        assert err <= LOGIT_TOL["bf16"], f"row {b}: logits {err:.3e} from the oracle"
    say(f"B={B} graph={graph}: {exact} of {B * (D + 1)} choices equal the oracle's exactly")
    assert len(set(toks.ravel().tolist())) > 1


def test_top_k_one_is_greedy(Q):
    W = S.make_weights(SHAPE, 53)
    ids = np.random.default_rng(54).integers(0, SHAPE.vocab, (2, 16)).astype(np.int32)
    m = Q.Model(SHAPE, Q.device_tensors(SHAPE, W), 2, 32)
    g_t, g_l = gpu_generate(m, ids, 6)
    m.set_sampling(0.7, 1, 1.0, 99)
    s_t, s_l = gpu_generate(m, ids, 6)
    m.close()
    assert np.array_equal(g_t, s_t) and np.array_equal(g_l, s_l)


def test_sampling_draws_alike_with_and_without_the_cache(Q):
    """The draw depends on (seed, row, position) only, so qw_generate with the
    cache and without it sample alike up to the first step whose choice lies
    at a boundary the two runs' rounding splits."""
    import torch
    W = S.make_weights(SHAPE, 55)
    B, P, D = 2, 20, 8
    ids = torch.from_numpy(np.random.default_rng(56).integers(0, SHAPE.vocab, (B, P)).astype(np.int32)).cuda()
    m = Q.Model(SHAPE, Q.device_tensors(SHAPE, W), B, P + D + 2)
    m.set_sampling(1.0, 40, 0.95, 7)
    lc = torch.empty((B, D + 1, SHAPE.vocab), dtype=torch.float32, device="cuda")
    lu = torch.empty_like(lc)
    tc = m.generate(ids, D, use_cache=True, logits=lc).cpu().numpy()
    tu = m.generate(ids, D, use_cache=False, logits=lu).cpu().numpy()
    m.close()
    lc, lu = lc.cpu().numpy(), lu.cpu().numpy()
    for b in range(B):
        diff = np.nonzero(tc[b] != tu[b])[0]
        k = int(diff[0]) if diff.size else D + 1
        assert np.abs(lc[b, :k] - lu[b, :k]).max() <= 2e-2 if k else True
        if diff.size:
            u = O.sampling_draw(7, b, P + k)
            check_choice(lu[b, k], int(tu[b, k]), 1.0, 40, 0.95, u, f"row {b} uncached at {k}")
            check_choice(lc[b, k], int(tc[b, k]), 1.0, 40, 0.95, u, f"row {b} cached at {k}")
        say(f"row {b}: cached and uncached sampled alike for {k} of {D + 1} steps")


@pytest.mark.parametrize("use_cache", [True, False])
def test_eos_finishes_a_sequence_on_the_device(Q, use_cache):
    """With eos set to a token row 0 emits greedily at step 3, row 0 emits it
    from there on; rows that never emit it are unchanged; the flags read
    back; a new prefill starts the sequences unfinished."""
    import torch
    W = S.make_weights(SHAPE, 57)
    B, P, D = 3, 18, 10
    ids_np = np.random.default_rng(58).integers(0, SHAPE.vocab, (B, P)).astype(np.int32)
    ids = torch.from_numpy(ids_np).cuda()
    m = Q.Model(SHAPE, Q.device_tensors(SHAPE, W), B, P + D + 2)
    ref = m.generate(ids, D, use_cache=use_cache).cpu().numpy()
    eos = int(ref[0, 3])
    m.set_eos(eos)
    got = m.generate(ids, D, use_cache=use_cache).cpu().numpy()
    fin = m.finished(B)
    for b in range(B):
        hits = np.nonzero(ref[b] == eos)[0]
        if hits.size == 0:
            assert np.array_equal(got[b], ref[b]) and fin[b] == 0
        else:
            f = int(hits[0])
            assert np.array_equal(got[b, :f + 1], ref[b, :f + 1])
            assert np.all(got[b, f:] == eos) and fin[b] == 1
    assert fin[0] == 1
    p_tok = m.prefill(ids).cpu().numpy()        # a new prefill starts unfinished, unless its token is eos
    assert m.finished(B) == [int(t == eos) for t in p_tok]
    m.set_eos(-1)
    assert m.finished(B) == [0] * B
    m.close()


def test_sampling_arguments(Q):
    m = Q.Model(SHAPE, Q.device_tensors(SHAPE, S.make_weights(SHAPE, 59)), 1, 16)
    for bad in ((0.0, 5, 1.0), (1.0, 1025, 1.0), (1.0, 5, 0.0), (1.0, 5, 1.5), (float("nan"), 5, 1.0)):
        with pytest.raises(Q.QwError) as e:
            m.set_sampling(*bad, seed=1)
        assert e.value.status == -1
    with pytest.raises(Q.QwError):
        m.set_eos(SHAPE.vocab)
    m.close()
