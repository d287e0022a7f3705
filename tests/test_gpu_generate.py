"""qw_generate: greedy generation with and without the KV cache ("augur":
cache benchmarking; "Building a Qwen2.5-1.5B Inference Engine From Scratch",
section 1.1: use_cache=False as ground truth)."""
import sys

import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests.helpers import assert_same_sequence, compare_row, gpu_generate

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


def generate(m, ids_np, steps, use_cache):
    import torch
    B, P = ids_np.shape
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    lg = torch.empty((B, steps + 1, m.shape.vocab), dtype=torch.float32, device="cuda")
    out = m.generate(ids, steps, use_cache=use_cache, logits=lg)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lg.cpu().numpy()


CASES = {
    # one row (fused decode kernels) and five rows (batched decode kernels)
    "hd128-b1": (S.ModelShape("g128", 2, 512, 4, 2, 128, 1536, 2049), 1, 40, 8),
    "hd64-g7-b5": (S.ModelShape("g64", 2, 448, 14, 2, 64, 896, 1100), 5, 30, 6),
}


@pytest.mark.parametrize("case", list(CASES))
def test_generate_cached_matches_decode_steps_and_uncached_matches_oracle(Q, case):
    shape, B, P, D = CASES[case]
    W = S.make_weights(shape, 41)
    ids = np.random.default_rng(42).integers(0, shape.vocab, (B, P)).astype(np.int32)
    m = Q.Model(shape, Q.device_tensors(shape, W), B, P + D + 4)
    ref_t, ref_l = gpu_generate(m, ids, D)                       # prefill + decode_step calls
    c_t, c_l = generate(m, ids, D, True)
    assert np.array_equal(c_t, ref_t) and np.array_equal(c_l, ref_l), "cached generation != decode steps"
    u_t, u_l = generate(m, ids, D, False)
    assert m.state() == (B, P + D)
    om = O.OracleModel(shape, W)
    for b in range(B):
        err, n = compare_row(om, ids[b], u_t[b], u_l[b], "bf16", f"{case} uncached row {b}")
        d = assert_same_sequence(c_t[b], c_l[b], u_t[b], u_l[b], label=f"{case} row {b} cached vs uncached")
        say(f"{case} row {b}: uncached vs oracle {err:.2e}, cached vs uncached {d:.2e}")
    # the cache an uncached run leaves behind continues with decode steps
    import torch
    nxt = torch.from_numpy(u_t[:, -1].copy()).cuda()
    lg = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
    m.decode_step(nxt, logits=lg)
    torch.cuda.synchronize()
    for b in range(B):
        ref = om.teacher_forced(ids[b], np.concatenate([u_t[b]]))[-1]
        assert np.abs(lg[b].cpu().numpy() - ref).max() <= 5e-2
    m.close()


def test_generate_errors(Q):
    import torch
    shape = S.ModelShape("gerr", 2, 256, 4, 2, 64, 512, 999)
    m = Q.Model(shape, Q.device_tensors(shape, S.make_weights(shape, 43)), 2, 16)
    ids = torch.zeros((2, 10), dtype=torch.int32, device="cuda")
    with pytest.raises(Q.QwError) as e:
        m.generate(ids, 7)                                          # 10 + 7 > 16
    assert e.value.status == -4
    with pytest.raises(Q.QwError) as e:
        m.generate(torch.zeros((3, 4), dtype=torch.int32, device="cuda"), 2)
    assert e.value.status == -1
    out = m.generate(ids, 6, use_cache=False)                       # exactly full
    torch.cuda.synchronize()
    assert out.shape == (2, 7) and m.state() == (2, 16)
    m.close()
