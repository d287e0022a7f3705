"""Paged KV cache and ragged batches ("augur", "Not yet" list: paged
attention, and batching of prompts of different lengths).

A paged model keeps each layer's cache as a pool of 64-position blocks with a
block table per sequence; its kernels do the same arithmetic as the dense
model's, so results must agree bit for bit.  A ragged prefill packs prompts
of different lengths without padding; each sequence is checked against the
oracle run on that sequence alone, and later decode steps continue every
sequence from its own position."""
import sys

import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests.helpers import LOGIT_TOL, compare_row, gpu_generate

pytestmark = pytest.mark.gpu

BLOCK = 64


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


def blocks(n):
    return (n + BLOCK - 1) // BLOCK


def ragged_generate(m, prompts, D, graph=True, noalloc=False):
    """qw_prefill_ragged, then D decode steps: tokens [n, D+1], logits [n, D+1, V]."""
    import torch
    n, V = len(prompts), m.shape.vocab
    lens = [len(p) for p in prompts]
    ids = torch.from_numpy(np.concatenate(prompts).astype(np.int32)).cuda()
    m.set_graph(graph)
    toks = torch.empty((D + 1, n), dtype=torch.int32, device="cuda")
    logits = torch.empty((D + 1, n, V), dtype=torch.float32, device="cuda")
    m.prefill_ragged(ids, lens, logits=logits[0], next_ids=toks[0])
    step = m.decode_step_noalloc if noalloc else m.decode_step
    for s in range(D):
        step(toks[s], logits=logits[s + 1], next_ids=toks[s + 1])
    torch.cuda.synchronize()
    return toks.cpu().numpy().T.copy(), logits.permute(1, 0, 2).cpu().numpy()


# (shape, batch, prompt, decode steps): each case crosses a block boundary
# while decoding and takes one of the decode attention kernels
PAGED = {
    # one row, short context: attention merged with the o projection
    "bf16-hd128-b1": (S.ModelShape("p128", 2, 512, 4, 2, 128, 1536, 2049), 1, 120, 12),
    # two rows past 256 keys: split-KV attention, partials merged in the o projection
    "bf16-hd128-b2-split": (S.ModelShape("p128", 2, 512, 4, 2, 128, 1536, 2049), 2, 300, 24),
    # more than two rows: split-KV attention on the matrix cores, batched projections
    "bf16-hd64-g7-b3": (S.ModelShape("p64g7", 2, 448, 14, 2, 64, 896, 1100), 3, 60, 10),
    # head dim 32: the vector-ALU split-KV attention
    "bf16-hd32-b3": (S.ModelShape("p32", 2, 256, 8, 2, 32, 640, 1000), 3, 62, 6),
    # fp32 weights: the generic kernels
    "f32-hd64-b2": (S.ModelShape("pf32", 2, 192, 6, 3, 64, 448, 513, dtype="f32"), 2, 61, 6),
}


@pytest.mark.parametrize("case", list(PAGED))
def test_paged_cache_matches_dense_bit_for_bit(Q, case):
    shape, B, P, D = PAGED[case]
    W = S.make_weights(shape, 71)
    ids = np.random.default_rng(72).integers(0, shape.vocab, (B, P)).astype(np.int32)
    smax = P + D + 3
    dense = Q.Model(shape, Q.device_tensors(shape, W), B, smax)
    t_d, l_d = gpu_generate(dense, ids, D)
    dense.close()
    need = B * blocks(P + D)
    paged = Q.Model(shape, Q.device_tensors(shape, W), B, smax, kv_blocks=need)
    assert paged.kv_blocks() == (need, need)
    t_p, l_p = gpu_generate(paged, ids, D)
    assert paged.kv_blocks() == (0, need)          # every block handed out, none twice
    assert paged.positions(B) == [P + D] * B
    paged.close()
    assert np.array_equal(t_d, t_p), f"{case}: tokens differ"
    assert np.array_equal(l_d, l_p), f"{case}: logits differ by up to {np.abs(l_d - l_p).max():.3e}"
    say(f"{case}: paged == dense over {D + 1} steps ({need} blocks)")


RAGGED = {
    # lengths around the 64-key tile and 128-query tile edges, one-token prompts
    "bf16-hd64-g7": (S.ModelShape("r64g7", 2, 448, 14, 2, 64, 896, 1100), [1, 63, 64, 65, 130, 7], 5),
    "bf16-hd128": (S.ModelShape("r128", 2, 512, 4, 2, 128, 1536, 2049), [200, 17, 129], 4),
    "f16-hd128-b2": (S.ModelShape("rh128", 2, 512, 4, 2, 128, 1536, 2049, dtype="f16"), [90, 33], 4),
    "bf16-hd32": (S.ModelShape("r32", 2, 256, 8, 2, 32, 640, 1000), [40, 3, 71], 4),
    "f32-hd64": (S.ModelShape("rf32", 2, 192, 6, 3, 64, 448, 513, dtype="f32"), [5, 21, 9], 4),
    # two rows, one past 256 keys: split-KV with the short row's later splits empty
    "bf16-hd64-split-b2": (S.ModelShape("rs64", 2, 256, 6, 2, 64, 512, 1001), [700, 20], 4),
    # three rows with split-KV over very different lengths
    "bf16-hd64-split-b3": (S.ModelShape("rs64", 2, 256, 6, 2, 64, 512, 1001), [300, 9, 650], 4),
}


@pytest.mark.parametrize("paged", [False, True], ids=["dense", "paged"])
@pytest.mark.parametrize("case", list(RAGGED))
def test_ragged_batch_matches_the_oracle(Q, case, paged):
    shape, lens, D = RAGGED[case]
    W = S.make_weights(shape, 73)
    rng = np.random.default_rng(74)
    prompts = [rng.integers(0, shape.vocab, n).astype(np.int32) for n in lens]
    n = len(lens)
    kw = {"kv_blocks": sum(blocks(x + D) for x in lens)} if paged else {}
    m = Q.Model(shape, Q.device_tensors(shape, W), n, max(lens) + D + 2, **kw)
    toks, logits = ragged_generate(m, prompts, D)
    assert m.positions(n) == [x + D for x in lens]
    assert m.state() == (n, max(lens) + D)
    m.close()
    om = O.OracleModel(shape, W)
    worst = 0.0
    for b in range(n):
        err, _ = compare_row(om, prompts[b], toks[b], logits[b], shape.dtype, f"{case} row {b} (len {lens[b]})")
        worst = max(worst, err)
    say(f"{case} {'paged' if paged else 'dense'}: lengths {lens}, max |dlogit| {worst:.3e}")


def test_ragged_equal_lengths_bit_identical_to_uniform(Q):
    """A ragged batch of equal lengths runs the same arithmetic as qw_prefill
    (only the order of the attention work items differs)."""
    shape = S.ModelShape("r64g7", 2, 448, 14, 2, 64, 896, 1100)
    W = S.make_weights(shape, 75)
    B, P, D = 3, 77, 4
    ids = np.random.default_rng(76).integers(0, shape.vocab, (B, P)).astype(np.int32)
    m = Q.Model(shape, Q.device_tensors(shape, W), B, P + D + 2)
    t_u, l_u = gpu_generate(m, ids, D)
    t_r, l_r = ragged_generate(m, list(ids), D)
    m.close()
    assert np.array_equal(t_u, t_r) and np.array_equal(l_u, l_r)


def test_ragged_paged_noalloc_step_matches(Q):
    """After a ragged prefill on a paged model the allocation-free step gives
    the captured step's results bit for bit (it takes blocks from the pool
    the same way)."""
    shape = S.ModelShape("r64g7", 2, 448, 14, 2, 64, 896, 1100)
    W = S.make_weights(shape, 77)
    rng = np.random.default_rng(78)
    lens, D = [62, 5, 127], 6
    prompts = [rng.integers(0, shape.vocab, x).astype(np.int32) for x in lens]
    nb = sum(blocks(x + D) for x in lens)
    m = Q.Model(shape, Q.device_tensors(shape, W), 3, 140, kv_blocks=nb)
    t_g, l_g = ragged_generate(m, prompts, D)
    t_n, l_n = ragged_generate(m, prompts, D, noalloc=True)
    assert m.kv_blocks() == (0, nb)
    m.close()
    assert np.array_equal(t_g, t_n) and np.array_equal(l_g, l_n)


def test_paged_pool_exhaustion_and_reuse(Q):
    """A prefill or a decode step that needs more blocks than the pool holds
    fails with CACHE_FULL before anything is enqueued; the state is unchanged
    and a smaller batch reuses the pool."""
    import torch
    shape = S.ModelShape("r64g7", 2, 448, 14, 2, 64, 896, 1100)
    W = S.make_weights(shape, 79)
    m = Q.Model(shape, Q.device_tensors(shape, W), 3, 256, kv_blocks=5)
    rng = np.random.default_rng(80)
    ids = torch.from_numpy(rng.integers(0, shape.vocab, (3, 128)).astype(np.int32)).cuda()
    with pytest.raises(Q.QwError) as e:
        m.prefill(ids)                                  # 3 x 2 blocks > 5
    assert e.value.status == -4
    assert m.state() == (0, 0)
    lens = [64, 128, 64]                               # 1 + 2 + 1 = 4 blocks
    packed = torch.from_numpy(rng.integers(0, shape.vocab, sum(lens)).astype(np.int32)).cuda()
    nxt = m.prefill_ragged(packed, lens)
    assert m.kv_blocks() == (1, 5)
    # every row starts a new block at the next step: 3 needed, 1 free
    with pytest.raises(Q.QwError) as e:
        m.decode_step(nxt)
    assert e.value.status == -4 and "block" in str(e.value)
    assert m.positions(3) == lens and m.kv_blocks() == (1, 5)
    # two rows fit: lengths 60 and 64 need 1 + 1 blocks, then one more at the step
    lens = [60, 64]
    packed = torch.from_numpy(rng.integers(0, shape.vocab, sum(lens)).astype(np.int32)).cuda()
    nxt = m.prefill_ragged(packed, lens)
    assert m.kv_blocks() == (3, 5)
    nxt = m.decode_step(nxt)
    assert m.kv_blocks() == (2, 5) and m.positions(2) == [61, 65]
    torch.cuda.synchronize()
    m.close()


def test_ragged_argument_errors(Q):
    import torch
    shape = S.ModelShape("r64g7", 2, 448, 14, 2, 64, 896, 1100)
    m = Q.Model(shape, Q.device_tensors(shape, S.make_weights(shape, 81)), 2, 64)
    ids = torch.zeros(70, dtype=torch.int32, device="cuda")
    for lens, status in (([0, 70], -1), ([65, 5], -4), ([10, 10, 10], -1)):
        with pytest.raises(Q.QwError) as e:
            m.prefill_ragged(ids[:sum(lens)], lens)
        assert e.value.status == status, lens
    assert m.state() == (0, 0)
    assert m.kv_blocks() == (0, 0)
    m.close()
