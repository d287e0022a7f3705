"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before touching HIP."""
import os
import re

import pytest

import synthetic as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def Q():
    import decoder_only_transformer_qwen2_amd as Q
    if not os.path.exists(Q.LIB_PATH):
        pytest.skip("libqw.so not built (run __graft_entry__.build())")
    Q.load_library()
    return Q


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qw.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qw_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("qw_create", "qw_prefill", "qw_decode_step", "qw_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol(Q):
    lib = Q.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(Q.EXPORTED) == set(declared_functions())


def test_kernel_family_names(Q):
    names = Q.qw_kernel_names()
    assert "gemm_gate_up" in names and "attention" in names and "mlp" in names
    assert len(names) == len(set(names))


def _cfg(Q, **kw):
    c = Q.make_config(S.TINY, 1, 64)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _weights(Q, n_layers=2):
    layers = (Q.qw_layer_weights * n_layers)()
    for l in range(n_layers):
        for f, _ in Q.qw_layer_weights._fields_:
            setattr(layers[l], f, 0x1000)          # never dereferenced: validation fails first
    return Q.qw_weights(0x1000, 0x1000, None, layers), layers


@pytest.mark.parametrize("field,value,status", [
    ("n_heads", 5, -1),            # not a multiple of n_kv_heads
    ("head_dim", 33, -1),          # odd head_dim
    ("head_dim", 48, -6),          # even, but not built
    ("hidden", 100, -6),           # not a multiple of 64
    ("n_layers", 0, -1),
    ("max_batch", 0, -1),
    ("qkv_bias", 0, -1),
    ("dtype", 7, -1),
    ("rope_theta", 0.0, -1),
])
def test_create_rejects_bad_config(Q, field, value, status):
    w, _keep = _weights(Q)
    with pytest.raises(Q.QwError) as e:
        Q.qw_create(_cfg(Q, **{field: value}), w, 0)
    assert e.value.status == status
    assert Q.qw_last_error()


def test_create_rejects_null_weights(Q):
    w, _keep = _weights(Q)
    w.embed = None
    with pytest.raises(Q.QwError) as e:
        Q.qw_create(_cfg(Q), w, 0)
    assert e.value.status == -1
    w, _keep = _weights(Q)
    _keep[1].down_w = None
    with pytest.raises(Q.QwError) as e:
        Q.qw_create(_cfg(Q), w, 0)
    assert "layer 1" in str(e.value)
    w, _keep = _weights(Q)
    with pytest.raises(Q.QwError) as e:
        Q.qw_create(_cfg(Q, tie_embeddings=0), w, 0)
    assert "lm_head" in str(e.value)


def test_calls_on_null_model(Q):
    lib = Q.load_library()
    assert lib.qw_prefill(None, None, 1, 1, None, 0, None) == -1
    assert lib.qw_decode_step(None, None, None, None) == -1
    assert lib.qw_prefill_ragged(None, None, None, 1, None, None) == -1
    assert lib.qw_get_positions(None, None, 0) == -1
    assert lib.qw_kv_blocks(None, None, None) == -1
    assert lib.qw_destroy(None) == 0


@pytest.mark.parametrize("blocks", [0, -3])
def test_create_paged_rejects_an_empty_pool(Q, blocks):
    w, _keep = _weights(Q)
    with pytest.raises(Q.QwError) as e:
        Q.qw_create_paged(_cfg(Q), w, blocks, 0)
    assert e.value.status == -1 and "num_blocks" in str(e.value)


def test_create_paged_validates_the_config_first(Q):
    w, _keep = _weights(Q)
    with pytest.raises(Q.QwError) as e:
        Q.qw_create_paged(_cfg(Q, n_heads=5), w, 8, 0)
    assert e.value.status == -1


def test_create_without_a_device_reports_the_hip_call(Q):
    """With no GPU the first HIP call of qw_create fails; the status is
    QW_ERR_HIP and the message still names the call after the half-built
    handle has been released."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the fake weight pointers must not reach a kernel")
    w, _keep = _weights(Q)
    with pytest.raises(Q.QwError) as e:
        Q.qw_create(_cfg(Q), w, 0)
    assert e.value.status == -3
    assert "hipStreamCreateWithFlags" in str(e.value)
    assert "hipStreamCreateWithFlags" in Q.qw_last_error()
