"""Python binding of libg4attn (batch-invariant hybrid GQA attention for MI355X).

Argument marshalling only: every step of the computation runs in the HIP kernels of
libg4attn.so. Tensors are torch tensors in device memory (bf16 as torch.bfloat16);
calls run asynchronously on torch's current stream unless a stream is given.
The functions carry the names of the C entry points declared in include/g4attn.h.
If the library has not been built, importing works but every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libg4attn.so")

G4ATTN_OK = 0
G4ATTN_ERR_INVALID_ARG = 1
G4ATTN_ERR_UNSUPPORTED = 2
G4ATTN_ERR_DEVICE = 3
G4ATTN_SLIDING = 0
G4ATTN_GLOBAL = 1
G4ATTN_ROPE_PAIRS_IN_BLOCK = 0
G4ATTN_ROPE_PAIRS_HALF_HEAD = 1

EXPORTED = ("g4attn_qk_prologue", "g4attn_prefill", "g4attn_prefill_qp", "g4attn_prefill_masked", "g4attn_prefill_cached",
            "g4attn_prefill_cached_masked", "g4attn_decode", "g4attn_prefill_backward",
            "g4attn_split_workspace_bytes", "g4attn_prefill_split", "g4attn_prefill_cached_split", "g4attn_decode_split",
            "g4attn_decode_split_noalloc", "g4attn_last_error",
            "g4attn_abi_version")


class Layer(ctypes.Structure):
    """Mirror of g4attn_layer."""

    _fields_ = [
        ("kind", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("k_eq_v", ctypes.c_int32),
        ("rope_dims", ctypes.c_int32),
        ("rope_freq_dim", ctypes.c_int32),
        ("rope_pairing", ctypes.c_int32),
        ("v_norm", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("softmax_scale", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
    ]


class Provenance(ctypes.Structure):
    """Mirror of g4attn_provenance."""

    _fields_ = [
        ("kernel_id", ctypes.c_char * 64),
        ("kind", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("block_q", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("mfma_m", ctypes.c_int32),
        ("mfma_n", ctypes.c_int32),
        ("mfma_k", ctypes.c_int32),
        ("waves_per_group", ctypes.c_int32),
        ("split_kv", ctypes.c_int32),
        ("acc_fp32", ctypes.c_int32),
        ("fallback", ctypes.c_int32),
        ("shape_fingerprint", ctypes.c_uint64),
    ]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["kernel_id"] = self.kernel_id.decode()
        return d


class G4AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"g4attn status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libg4attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.g4attn_qk_prologue.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]
        L.g4attn_qk_prologue.restype = i32
        L.g4attn_prefill.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, i32, i32, vp, ctypes.POINTER(Provenance)]
        L.g4attn_prefill.restype = i32
        L.g4attn_prefill_qp.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp,
                                        ctypes.POINTER(Provenance)]
        L.g4attn_prefill_qp.restype = i32
        L.g4attn_prefill_masked.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, vp, i32, i32, vp,
                                            ctypes.POINTER(Provenance)]
        L.g4attn_prefill_masked.restype = i32
        L.g4attn_prefill_cached.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                            i32, vp, ctypes.POINTER(Provenance)]
        L.g4attn_prefill_cached.restype = i32
        L.g4attn_prefill_cached_masked.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                                   i32, i32, vp, ctypes.POINTER(Provenance)]
        L.g4attn_prefill_cached_masked.restype = i32
        L.g4attn_decode.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, vp,
                                    ctypes.POINTER(Provenance)]
        L.g4attn_decode.restype = i32
        L.g4attn_prefill_backward.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              i32, i32, vp]
        L.g4attn_prefill_backward.restype = i32
        u64 = ctypes.c_uint64
        L.g4attn_split_workspace_bytes.argtypes = [ctypes.POINTER(Layer), i32, i32, i32, i32, ctypes.POINTER(u64)]
        L.g4attn_split_workspace_bytes.restype = i32
        L.g4attn_prefill_split.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, u64, vp,
                                           ctypes.POINTER(Provenance)]
        L.g4attn_prefill_split.restype = i32
        L.g4attn_prefill_cached_split.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                                  i32, i32, vp, u64, vp, ctypes.POINTER(Provenance)]
        L.g4attn_prefill_cached_split.restype = i32
        L.g4attn_decode_split.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, i32, vp,
                                          u64, vp, ctypes.POINTER(Provenance)]
        L.g4attn_decode_split.restype = i32
        L.g4attn_decode_split_noalloc.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, i32,
                                                  vp, ctypes.POINTER(Provenance)]
        L.g4attn_decode_split_noalloc.restype = i32
        L.g4attn_last_error.argtypes = []
        L.g4attn_last_error.restype = ctypes.c_char_p
        L.g4attn_abi_version.argtypes = []
        L.g4attn_abi_version.restype = i32
        _lib = L
    return _lib


def g4attn_last_error() -> str:
    return lib().g4attn_last_error().decode()


def g4attn_abi_version() -> int:
    return int(lib().g4attn_abi_version())


def make_layer(spec) -> Layer:
    """g4attn_layer from any object with the LayerSpec attributes (see workloads)."""
    return Layer(kind=int(spec.kind), num_q_heads=spec.num_q_heads, num_kv_heads=spec.num_kv_heads,
                 head_dim=spec.head_dim, window=spec.window, k_eq_v=int(bool(spec.k_eq_v)),
                 rope_dims=spec.rope_dims, rope_freq_dim=spec.rope_freq_dim,
                 rope_pairing=int(getattr(spec, "rope_pairing", G4ATTN_ROPE_PAIRS_IN_BLOCK)),
                 v_norm=int(bool(getattr(spec, "v_norm", False))),
                 rope_theta=float(spec.rope_theta), softmax_scale=float(spec.softmax_scale),
                 rms_eps=float(spec.rms_eps))


def _check(status: int) -> None:
    if status != G4ATTN_OK:
        raise G4AttnError(status, g4attn_last_error())


def _ptr(t, dtype=None) -> Optional[int]:
    if t is None:
        return None
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(t)}")
    if not t.is_cuda:
        raise ValueError("tensors must be in device memory")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def g4attn_qk_prologue(layer: Layer, q_in, q_out, k_in, k_out, q_norm_w, k_norm_w, positions,
                       v_in=None, v_out=None, kv_dst_row=None, num_tokens: Optional[int] = None,
                       stream=None) -> None:
    import torch

    bf, i32, i64 = torch.bfloat16, torch.int32, torch.int64
    if num_tokens is None:
        num_tokens = int(positions.shape[0])
    _check(lib().g4attn_qk_prologue(ctypes.byref(layer), _ptr(q_in, bf), _ptr(q_out, bf), _ptr(k_in, bf),
                                    _ptr(k_out, bf), _ptr(v_in, bf), _ptr(v_out, bf), _ptr(q_norm_w, bf),
                                    _ptr(k_norm_w, bf), _ptr(positions, i32), _ptr(kv_dst_row, i64),
                                    int(num_tokens), _stream(stream)))


def g4attn_prefill(layer: Layer, q, k, v, out, seq_start, seq_len, max_seq_len: int, stream=None,
                   provenance: bool = False):
    import torch

    bf, i32 = torch.bfloat16, torch.int32
    prov = Provenance() if provenance else None
    _check(lib().g4attn_prefill(ctypes.byref(layer), _ptr(q, bf), _ptr(k, bf), _ptr(v, bf), _ptr(out, bf),
                                _ptr(seq_start, i32), _ptr(seq_len, i32), int(seq_len.shape[0]), int(max_seq_len),
                                _stream(stream), ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None


def g4attn_prefill_qp(layer: Layer, q, q_norm_w, positions, k, v, out, seq_start, seq_len, max_seq_len: int,
                      stream=None, provenance: bool = False):
    """g4attn_prefill of raw q rows, the q prologue inside (head dim 512, K=V)."""
    import torch

    bf, i32 = torch.bfloat16, torch.int32
    prov = Provenance() if provenance else None
    _check(lib().g4attn_prefill_qp(ctypes.byref(layer), _ptr(q, bf), _ptr(q_norm_w, bf), _ptr(positions, i32),
                                   _ptr(k, bf), _ptr(v, bf), _ptr(out, bf), _ptr(seq_start, i32),
                                   _ptr(seq_len, i32), int(seq_len.shape[0]), int(max_seq_len), _stream(stream),
                                   ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None


def g4attn_prefill_masked(layer: Layer, q, k, v, out, seq_start, seq_len, last_key, max_seq_len: int, stream=None,
                          provenance: bool = False):
    import torch

    bf, i32 = torch.bfloat16, torch.int32
    prov = Provenance() if provenance else None
    _check(lib().g4attn_prefill_masked(ctypes.byref(layer), _ptr(q, bf), _ptr(k, bf), _ptr(v, bf), _ptr(out, bf),
                                       _ptr(seq_start, i32), _ptr(seq_len, i32), _ptr(last_key, i32),
                                       int(seq_len.shape[0]), int(max_seq_len), _stream(stream),
                                       ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None


def g4attn_prefill_cached(layer: Layer, q, k_cache, v_cache, out, q_row0, q_pos0, chunk_len, cache_row0,
                          cache_slots: int, max_chunk_len: int, max_key_len: int, stream=None,
                          provenance: bool = False):
    import torch

    bf, i32, i64 = torch.bfloat16, torch.int32, torch.int64
    prov = Provenance() if provenance else None
    _check(lib().g4attn_prefill_cached(ctypes.byref(layer), _ptr(q, bf), _ptr(k_cache, bf), _ptr(v_cache, bf),
                                       _ptr(out, bf), _ptr(q_row0, i32), _ptr(q_pos0, i32), _ptr(chunk_len, i32),
                                       _ptr(cache_row0, i64), int(cache_slots), int(chunk_len.shape[0]),
                                       int(max_chunk_len), int(max_key_len), _stream(stream),
                                       ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None


def g4attn_prefill_cached_masked(layer: Layer, q, k_cache, v_cache, out, q_row0, q_pos0, chunk_len, last_key,
                                 cache_row0, cache_slots: int, max_chunk_len: int, max_key_len: int, stream=None,
                                 provenance: bool = False):
    import torch

    bf, i32, i64 = torch.bfloat16, torch.int32, torch.int64
    prov = Provenance() if provenance else None
    _check(lib().g4attn_prefill_cached_masked(ctypes.byref(layer), _ptr(q, bf), _ptr(k_cache, bf),
                                              _ptr(v_cache, bf), _ptr(out, bf), _ptr(q_row0, i32), _ptr(q_pos0, i32),
                                              _ptr(chunk_len, i32), _ptr(last_key, i32), _ptr(cache_row0, i64),
                                              int(cache_slots), int(chunk_len.shape[0]), int(max_chunk_len),
                                              int(max_key_len), _stream(stream),
                                              ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None


def g4attn_decode(layer: Layer, q, k_cache, v_cache, cache_row0, ctx_len, cache_slots: int, out,
                  max_ctx_len: int, schedule=None, stream=None, provenance: bool = False):
    import torch

    bf, i32, i64 = torch.bfloat16, torch.int32, torch.int64
    prov = Provenance() if provenance else None
    _check(lib().g4attn_decode(ctypes.byref(layer), _ptr(q, bf), _ptr(k_cache, bf), _ptr(v_cache, bf),
                               _ptr(cache_row0, i64), _ptr(ctx_len, i32), int(cache_slots), _ptr(out, bf),
                               int(ctx_len.shape[0]), int(max_ctx_len), _ptr(schedule, i32), _stream(stream),
                               ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None


def g4attn_prefill_backward(layer: Layer, q, k, v, out, dout, dq, dk, dv, lse, delta, seq_start, seq_len,
                            max_seq_len: int, stream=None) -> None:
    import torch

    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _check(lib().g4attn_prefill_backward(ctypes.byref(layer), _ptr(q, bf), _ptr(k, bf), _ptr(v, bf), _ptr(out, bf),
                                         _ptr(dout, bf), _ptr(dq, bf), _ptr(dk, bf), _ptr(dv, bf), _ptr(lse, f32),
                                         _ptr(delta, f32), _ptr(seq_start, i32), _ptr(seq_len, i32),
                                         int(seq_len.shape[0]), int(max_seq_len), _stream(stream)))


def g4attn_split_workspace_bytes(layer: Layer, batch: int, rows: int, max_key_len: int, split_keys: int) -> int:
    n = ctypes.c_uint64(0)
    _check(lib().g4attn_split_workspace_bytes(ctypes.byref(layer), int(batch), int(rows), int(max_key_len),
                                              int(split_keys), ctypes.byref(n)))
    return int(n.value)


def _workspace(ws):
    """(pointer, bytes) of a workspace tensor in device memory (any dtype), or (None, 0)."""
    if ws is None:
        return None, 0
    return _ptr(ws), int(ws.numel()) * int(ws.element_size())


def g4attn_prefill_split(layer: Layer, q, k, v, out, seq_start, seq_len, max_seq_len: int, split_keys: int,
                         workspace, stream=None, provenance: bool = False):
    import torch

    bf, i32 = torch.bfloat16, torch.int32
    prov = Provenance() if provenance else None
    wp, wb = _workspace(workspace)
    _check(lib().g4attn_prefill_split(ctypes.byref(layer), _ptr(q, bf), _ptr(k, bf), _ptr(v, bf), _ptr(out, bf),
                                      _ptr(seq_start, i32), _ptr(seq_len, i32), int(seq_len.shape[0]),
                                      int(max_seq_len), int(split_keys), wp, wb, _stream(stream),
                                      ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None


def g4attn_prefill_cached_split(layer: Layer, q, k_cache, v_cache, out, q_row0, q_pos0, chunk_len, cache_row0,
                                cache_slots: int, max_chunk_len: int, max_key_len: int, split_keys: int, workspace,
                                stream=None, provenance: bool = False):
    import torch

    bf, i32, i64 = torch.bfloat16, torch.int32, torch.int64
    prov = Provenance() if provenance else None
    wp, wb = _workspace(workspace)
    _check(lib().g4attn_prefill_cached_split(ctypes.byref(layer), _ptr(q, bf), _ptr(k_cache, bf), _ptr(v_cache, bf),
                                             _ptr(out, bf), _ptr(q_row0, i32), _ptr(q_pos0, i32),
                                             _ptr(chunk_len, i32), _ptr(cache_row0, i64), int(cache_slots),
                                             int(chunk_len.shape[0]), int(max_chunk_len), int(max_key_len),
                                             int(split_keys), wp, wb, _stream(stream),
                                             ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None


def g4attn_decode_split(layer: Layer, q, k_cache, v_cache, cache_row0, ctx_len, cache_slots: int, out,
                        max_ctx_len: int, split_keys: int, workspace, schedule=None, stream=None,
                        provenance: bool = False):
    import torch

    bf, i32, i64 = torch.bfloat16, torch.int32, torch.int64
    prov = Provenance() if provenance else None
    wp, wb = _workspace(workspace)
    _check(lib().g4attn_decode_split(ctypes.byref(layer), _ptr(q, bf), _ptr(k_cache, bf), _ptr(v_cache, bf),
                                     _ptr(cache_row0, i64), _ptr(ctx_len, i32), int(cache_slots), _ptr(out, bf),
                                     int(ctx_len.shape[0]), int(max_ctx_len), _ptr(schedule, i32), int(split_keys),
                                     wp, wb, _stream(stream), ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None


def g4attn_decode_split_noalloc(layer: Layer, q, k_cache, v_cache, cache_row0, ctx_len, cache_slots: int, out,
                                max_ctx_len: int, split_keys: int, schedule=None, stream=None,
                                provenance: bool = False):
    import torch

    bf, i32, i64 = torch.bfloat16, torch.int32, torch.int64
    prov = Provenance() if provenance else None
    _check(lib().g4attn_decode_split_noalloc(ctypes.byref(layer), _ptr(q, bf), _ptr(k_cache, bf), _ptr(v_cache, bf),
                                             _ptr(cache_row0, i64), _ptr(ctx_len, i32), int(cache_slots),
                                             _ptr(out, bf), int(ctx_len.shape[0]), int(max_ctx_len),
                                             _ptr(schedule, i32), int(split_keys), _stream(stream),
                                             ctypes.byref(prov) if prov is not None else None))
    return prov.as_dict() if prov is not None else None
