"""ctypes binding of libqw.so (include/qw.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of libqw.so.  The functions below carry the C names and take device
pointers as Python ints; `Model` is a convenience wrapper that keeps the
torch tensors alive and passes their `data_ptr()`s.  If the library has not
been built, loading it raises -- there is no other execution path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# QW_LIB names another build of the same library (e.g. to compare two builds)
LIB_PATH = os.environ.get("QW_LIB") or os.path.join(_PKG, "libqw.so")

QW_OK, QW_ERR_INVALID_ARG, QW_ERR_OUT_OF_MEMORY, QW_ERR_HIP = 0, -1, -2, -3
QW_ERR_CACHE_FULL, QW_ERR_BAD_STATE, QW_ERR_UNSUPPORTED, QW_ERR_NUMERICS = -4, -5, -6, -7
QW_F32, QW_BF16, QW_F16 = 0, 1, 2

STATUS_NAMES = {0: "QW_OK", -1: "QW_ERR_INVALID_ARG", -2: "QW_ERR_OUT_OF_MEMORY", -3: "QW_ERR_HIP",
                -4: "QW_ERR_CACHE_FULL", -5: "QW_ERR_BAD_STATE", -6: "QW_ERR_UNSUPPORTED",
                -7: "QW_ERR_NUMERICS"}

EXPORTED = ("qw_create", "qw_create_paged", "qw_prefill", "qw_prefill_ragged", "qw_decode_step",
            "qw_decode_step_noalloc", "qw_generate", "qw_destroy", "qw_last_error", "qw_get_state",
            "qw_get_positions", "qw_kv_blocks", "qw_check_ids", "qw_check_numerics", "qw_set_sampling",
            "qw_set_eos", "qw_get_finished", "qw_set_graph", "qw_timing_enable", "qw_timing_read",
            "qw_kernel_names", "qw_peak_copy", "qw_peak_mfma")

QW_KV_BLOCK = 64


class QwError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class qw_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("qkv_bias", ctypes.c_int32), ("tie_embeddings", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("max_seq", ctypes.c_int32)]


class qw_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("input_norm", "q_w", "q_b", "k_w", "k_b", "v_w", "v_b", "o_w",
                                              "post_norm", "gate_w", "up_w", "down_w")]


class qw_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(qw_layer_weights))]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqw.so (once).  Raises if it is missing: build it first with
    `python -m decoder_only_transformer_qwen2_amd.build`."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m decoder_only_transformer_qwen2_amd.build`")
    # torch ships its own HIP runtime; loading it first makes libqw.so bind to
    # that same runtime (one HIP runtime per process, shared streams)
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "qw_create": (I32, [ctypes.POINTER(qw_config), ctypes.POINTER(qw_weights), P, ctypes.POINTER(P)]),
        "qw_create_paged": (I32, [ctypes.POINTER(qw_config), ctypes.POINTER(qw_weights), I32, P,
                                  ctypes.POINTER(P)]),
        "qw_prefill": (I32, [P, P, I32, I32, P, I32, P]),
        "qw_prefill_ragged": (I32, [P, P, ctypes.POINTER(I32), I32, P, P]),
        "qw_get_positions": (I32, [P, ctypes.POINTER(I32), I32]),
        "qw_kv_blocks": (I32, [P, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "qw_decode_step": (I32, [P, P, P, P]),
        "qw_decode_step_noalloc": (I32, [P, P, P, P]),
        "qw_generate": (I32, [P, P, I32, I32, I32, I32, P, P]),
        "qw_destroy": (I32, [P]),
        "qw_last_error": (ctypes.c_char_p, []),
        "qw_get_state": (I32, [P, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "qw_check_ids": (I32, [P]),
        "qw_check_numerics": (I32, [P]),
        "qw_set_sampling": (I32, [P, ctypes.c_float, I32, ctypes.c_float, ctypes.c_uint64]),
        "qw_set_eos": (I32, [P, I32]),
        "qw_get_finished": (I32, [P, ctypes.POINTER(I32), I32]),
        "qw_set_graph": (I32, [P, I32]),
        "qw_timing_enable": (I32, [P, ctypes.c_char_p]),
        "qw_timing_read": (I32, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64), I32]),
        "qw_kernel_names": (ctypes.c_char_p, []),
        "qw_peak_copy": (I32, [P, P, I64, I32, I32, P, ctypes.POINTER(ctypes.c_double)]),
        "qw_peak_mfma": (I32, [I32, P, ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != QW_OK:
        raise QwError(status, qw_last_error())


# ---------------------------------------------------------------- thin C-named wrappers
def qw_last_error() -> str:
    return load_library().qw_last_error().decode()


def qw_kernel_names() -> list:
    return load_library().qw_kernel_names().decode().split(",")


def qw_create(cfg: qw_config, weights: qw_weights, stream: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(load_library().qw_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.c_void_p(stream),
                                    ctypes.byref(h)))
    return h.value


def qw_create_paged(cfg: qw_config, weights: qw_weights, num_blocks: int, stream: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(load_library().qw_create_paged(ctypes.byref(cfg), ctypes.byref(weights), num_blocks,
                                          ctypes.c_void_p(stream), ctypes.byref(h)))
    return h.value


def qw_prefill(model: int, ids: int, batch: int, prompt_len: int, logits: int, logits_all: int,
               next_ids: int) -> None:
    _check(load_library().qw_prefill(model, ids, batch, prompt_len, logits or None, logits_all, next_ids))


def qw_prefill_ragged(model: int, ids: int, lens, logits: int, next_ids: int) -> None:
    """lens: host sequence of prompt lengths (ids holds the prompts packed)."""
    n = len(lens)
    buf = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in lens])
    _check(load_library().qw_prefill_ragged(model, ids, buf, n, logits or None, next_ids))


def qw_get_positions(model: int, n: int) -> list:
    buf = (ctypes.c_int32 * max(n, 1))()
    _check(load_library().qw_get_positions(model, buf, n))
    return [int(buf[i]) for i in range(n)]


def qw_kv_blocks(model: int):
    f, t = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().qw_kv_blocks(model, ctypes.byref(f), ctypes.byref(t)))
    return f.value, t.value


def qw_decode_step(model: int, ids: int, logits: int, next_ids: int) -> None:
    _check(load_library().qw_decode_step(model, ids, logits or None, next_ids))


def qw_decode_step_noalloc(model: int, ids: int, logits: int, next_ids: int) -> None:
    _check(load_library().qw_decode_step_noalloc(model, ids, logits or None, next_ids))


def qw_generate(model: int, ids: int, batch: int, prompt_len: int, steps: int, use_cache: bool, out_ids: int,
                logits: int) -> None:
    _check(load_library().qw_generate(model, ids, batch, prompt_len, steps, int(bool(use_cache)), out_ids,
                                      logits or None))


def qw_destroy(model: int) -> None:
    _check(load_library().qw_destroy(model))


def qw_get_state(model: int):
    b, p = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().qw_get_state(model, ctypes.byref(b), ctypes.byref(p)))
    return b.value, p.value


def qw_check_ids(model: int) -> None:
    _check(load_library().qw_check_ids(model))


def qw_check_numerics(model: int) -> None:
    _check(load_library().qw_check_numerics(model))


def qw_set_sampling(model: int, temperature: float, top_k: int, top_p: float, seed: int) -> None:
    _check(load_library().qw_set_sampling(model, temperature, top_k, top_p, seed))


def qw_set_eos(model: int, eos_id: int) -> None:
    _check(load_library().qw_set_eos(model, eos_id))


def qw_get_finished(model: int, n: int) -> list:
    buf = (ctypes.c_int32 * max(n, 1))()
    _check(load_library().qw_get_finished(model, buf, n))
    return [int(buf[i]) for i in range(n)]


def qw_set_graph(model: int, enable: bool) -> None:
    _check(load_library().qw_set_graph(model, int(bool(enable))))


def qw_timing_enable(model: int, name: Optional[str]) -> None:
    _check(load_library().qw_timing_enable(model, name.encode() if name else None))


def qw_timing_read(model: int, reset: bool = True):
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(load_library().qw_timing_read(model, ctypes.byref(ms), ctypes.byref(n), int(reset)))
    return ms.value, n.value


def qw_peak_copy(dst: int, src: int, nbytes: int, iters: int, read_only: bool = False, stream: int = 0) -> float:
    """HBM rate in GB/s of a copy (bytes read + written per second / 1e9) or,
    with read_only, of a pass that reads every byte once."""
    r = ctypes.c_double()
    _check(load_library().qw_peak_copy(dst, src, nbytes, iters, int(bool(read_only)), ctypes.c_void_p(stream),
                                       ctypes.byref(r)))
    return r.value


def qw_peak_mfma(iters: int, stream: int = 0) -> float:
    """Dense fp16 MFMA rate in TFLOP/s of an MFMA-only loop."""
    r = ctypes.c_double()
    _check(load_library().qw_peak_mfma(iters, ctypes.c_void_p(stream), ctypes.byref(r)))
    return r.value


# ---------------------------------------------------------------- convenience wrapper
_LAYER_KEYS = {
    "input_norm": "input_layernorm.weight", "q_w": "self_attn.q_proj.weight", "q_b": "self_attn.q_proj.bias",
    "k_w": "self_attn.k_proj.weight", "k_b": "self_attn.k_proj.bias", "v_w": "self_attn.v_proj.weight",
    "v_b": "self_attn.v_proj.bias", "o_w": "self_attn.o_proj.weight",
    "post_norm": "post_attention_layernorm.weight", "gate_w": "mlp.gate_proj.weight",
    "up_w": "mlp.up_proj.weight", "down_w": "mlp.down_proj.weight",
}


def make_config(shape, max_batch: int, max_seq: int) -> qw_config:
    """qw_config from any object with the ModelShape field names."""
    return qw_config(shape.n_layers, shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                     shape.intermediate, shape.vocab, shape.rms_eps, shape.rope_theta, 1,
                     int(shape.tie_embeddings), {"bf16": QW_BF16, "f16": QW_F16, "f32": QW_F32}[shape.dtype],
                     max_batch, max_seq)


class Model:
    """A libqw model built from device tensors keyed by HF Qwen2 names.

    `tensors` values are torch CUDA tensors (torch.bfloat16, torch.float16 or
    torch.float32 as the shape's dtype says), contiguous, in HF [out, in]
    layouts.  The
    library copies what it needs at creation, so they may be dropped after.
    """

    def __init__(self, shape, tensors: Dict[str, "object"], max_batch: int, max_seq: int, stream=None,
                 kv_blocks: Optional[int] = None):
        """kv_blocks: a paged cache of that many QW_KV_BLOCK-position blocks
        (qw_create_paged) instead of the dense max_batch x max_seq one."""
        import torch
        self.shape = shape
        self.cfg = make_config(shape, max_batch, max_seq)
        want = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[shape.dtype]
        for k, t in tensors.items():
            if t.dtype != want or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{k}: need a contiguous CUDA {want} tensor")
        layers = (qw_layer_weights * shape.n_layers)()
        for l in range(shape.n_layers):
            for f, key in _LAYER_KEYS.items():
                setattr(layers[l], f, tensors[f"model.layers.{l}.{key}"].data_ptr())
        w = qw_weights(tensors["model.embed_tokens.weight"].data_ptr(), tensors["model.norm.weight"].data_ptr(),
                       tensors["lm_head.weight"].data_ptr() if "lm_head.weight" in tensors else None, layers)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        if kv_blocks is None:
            self.handle = qw_create(self.cfg, w, self.stream.cuda_stream)
        else:
            self.handle = qw_create_paged(self.cfg, w, kv_blocks, self.stream.cuda_stream)

    def prefill(self, ids, logits=None, logits_all: bool = False, next_ids=None):
        import torch
        B, P = ids.shape
        if next_ids is None:
            next_ids = torch.empty(B, dtype=torch.int32, device=ids.device)
        qw_prefill(self.handle, ids.data_ptr(), B, P, logits.data_ptr() if logits is not None else 0,
                   int(logits_all), next_ids.data_ptr())
        return next_ids

    def prefill_ragged(self, ids, lens, logits=None, next_ids=None):
        """ids: int32 CUDA tensor of the prompts packed back to back; lens:
        their lengths (host ints)."""
        import torch
        lens = [int(x) for x in lens]
        if ids.numel() != sum(lens):
            raise ValueError(f"ids holds {ids.numel()} tokens, lens sum to {sum(lens)}")
        if next_ids is None:
            next_ids = torch.empty(len(lens), dtype=torch.int32, device=ids.device)
        qw_prefill_ragged(self.handle, ids.data_ptr(), lens, logits.data_ptr() if logits is not None else 0,
                          next_ids.data_ptr())
        return next_ids

    def positions(self, n: int):
        return qw_get_positions(self.handle, n)

    def kv_blocks(self):
        """(free, total) blocks of a paged cache; (0, 0) when dense."""
        return qw_kv_blocks(self.handle)

    def decode_step(self, ids, logits=None, next_ids=None):
        import torch
        if next_ids is None:
            next_ids = torch.empty(ids.shape[0], dtype=torch.int32, device=ids.device)
        qw_decode_step(self.handle, ids.data_ptr(), logits.data_ptr() if logits is not None else 0,
                       next_ids.data_ptr())
        return next_ids

    def decode_step_noalloc(self, ids, logits=None, next_ids=None):
        import torch
        if next_ids is None:
            next_ids = torch.empty(ids.shape[0], dtype=torch.int32, device=ids.device)
        qw_decode_step_noalloc(self.handle, ids.data_ptr(), logits.data_ptr() if logits is not None else 0,
                               next_ids.data_ptr())
        return next_ids

    def generate(self, ids, steps: int, use_cache: bool = True, logits=None, out_ids=None):
        """Greedy tokens [B, steps + 1] (and logits [B, steps + 1, V] if a
        buffer is given) with or without the KV cache."""
        import torch
        B, P = ids.shape
        if out_ids is None:
            out_ids = torch.empty((B, steps + 1), dtype=torch.int32, device=ids.device)
        qw_generate(self.handle, ids.data_ptr(), B, P, steps, use_cache, out_ids.data_ptr(),
                    logits.data_ptr() if logits is not None else 0)
        return out_ids

    def state(self):
        return qw_get_state(self.handle)

    def check_ids(self):
        qw_check_ids(self.handle)

    def check_numerics(self):
        qw_check_numerics(self.handle)

    def set_sampling(self, temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0, seed: int = 0):
        qw_set_sampling(self.handle, temperature, top_k, top_p, seed)

    def set_eos(self, eos_id: int):
        qw_set_eos(self.handle, eos_id)

    def finished(self, n: int):
        return qw_get_finished(self.handle, n)

    def set_graph(self, enable: bool):
        qw_set_graph(self.handle, enable)

    def timing_enable(self, name: Optional[str]):
        qw_timing_enable(self.handle, name)

    def timing_read(self, reset: bool = True):
        return qw_timing_read(self.handle, reset)

    def close(self):
        if getattr(self, "handle", None):
            qw_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def device_tensors(shape, weights: Dict[str, "object"], device="cuda"):
    """Move seeded numpy weights (uint16 bf16 bit patterns, float16 or
    float32) to the device as torch tensors of the matching dtype (a
    bit-exact copy)."""
    import numpy as np
    import torch
    out = {}
    for k, a in weights.items():
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        elif a.dtype == np.float16:
            t = torch.from_numpy(np.ascontiguousarray(a))
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        out[k] = t.to(device).contiguous()
    return out
