"""qw_decode_step_noalloc (for callers that cannot allocate) against
qw_decode_step: same tokens and logits, bit for bit, on consecutive calls of
which the second has a smaller batch (the static scratch array keeps the
larger call's contents)."""
import numpy as np
import pytest

import synthetic as S
from tests.helpers import gpu_generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_only_transformer_qwen2_amd as Q
    Q.load_library()
    return Q


def noalloc_generate(model, ids_np, steps):
    import torch
    B = ids_np.shape[0]
    V = model.shape.vocab
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    toks = torch.empty((steps + 1, B), dtype=torch.int32, device="cuda")
    logits = torch.empty((steps + 1, B, V), dtype=torch.float32, device="cuda")
    model.prefill(ids, logits=logits[0], next_ids=toks[0])
    for s in range(steps):
        model.decode_step_noalloc(toks[s], logits=logits[s + 1], next_ids=toks[s + 1])
    torch.cuda.synchronize()
    return toks.cpu().numpy().T.copy(), logits.permute(1, 0, 2).cpu().numpy()


# (model, rows of the larger call, rows of the smaller call, prompt, steps)
CASES = {
    # 5 rows: norm kernel + batched projections + split-KV attention; then
    # 2 rows: fused norms, merged attention + o projection, one-kernel MLP
    "hd64-g7": (S.ModelShape("na64", 2, 448, 14, 2, 64, 896, 1100), 5, 2, 40, 6),
    # the 1.5B widths: 3 rows, then one row past 256 keys (split-KV pair)
    "h1536": (S.ModelShape("na1536", 2, 1536, 12, 2, 128, 8960, 3001), 3, 1, 258, 4),
}


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_step_matches_decode_step(Q, case):
    shape, b_big, b_small, P, D = CASES[case]
    W = S.make_weights(shape, 31)
    rng = np.random.default_rng(32)
    ids_big = rng.integers(0, shape.vocab, (b_big, P)).astype(np.int32)
    ids_small = rng.integers(0, shape.vocab, (b_small, P)).astype(np.int32)
    m = Q.Model(shape, Q.device_tensors(shape, W), b_big, P + D + 2)
    ref_big = gpu_generate(m, ids_big, D, graph=False)
    ref_small = gpu_generate(m, ids_small, D, graph=False)
    got_big = noalloc_generate(m, ids_big, D)
    got_small = noalloc_generate(m, ids_small, D)     # right after the larger call
    m.close()
    for ref, got, label in ((ref_big, got_big, f"{b_big} rows"), (ref_small, got_small, f"{b_small} rows")):
        assert np.array_equal(ref[0], got[0]), f"{case} {label}: tokens differ"
        assert np.array_equal(ref[1], got[1]), f"{case} {label}: logits differ " \
                                               f"(max {np.abs(ref[1] - got[1]).max():.3e})"


def test_noalloc_step_errors(Q):
    import torch
    shape = S.ModelShape("na_err", 2, 256, 4, 2, 64, 512, 999)
    m = Q.Model(shape, Q.device_tensors(shape, S.make_weights(shape, 33)), 2, 8)
    nxt = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(Q.QwError) as e:
        m.decode_step_noalloc(nxt, next_ids=nxt)
    assert e.value.status == -5                              # BAD_STATE: no prefill
    ids = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    m.prefill(ids, next_ids=nxt)
    with pytest.raises(Q.QwError) as e:
        m.decode_step_noalloc(nxt, next_ids=nxt)
    assert e.value.status == -4                              # CACHE_FULL
    m.close()
    f32 = S.ModelShape("na_f32", 2, 128, 4, 2, 32, 256, 500, dtype="f32")
    m = Q.Model(f32, Q.device_tensors(f32, S.make_weights(f32, 34)), 1, 16)
    ids = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    nxt = m.prefill(ids)
    with pytest.raises(Q.QwError) as e:
        m.decode_step_noalloc(nxt, next_ids=nxt)
    assert e.value.status == -6                              # UNSUPPORTED: generic step
    m.close()
