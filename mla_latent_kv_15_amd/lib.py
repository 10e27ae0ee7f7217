"""Thin ctypes binding of libmla.so (include/mla.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device memory (``tensor.data_ptr()``) and the current HIP
stream.  Loading fails loudly when the library has not been built; there is
no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, or another build of the same library named by MLA_LIBRARY
# (the sanitized host build, for instance)
LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(_HERE, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4
MLA_ERR_SCRATCH_LIMIT = -5

MLA_F32 = 0
MLA_BF16 = 1

OP_APPEND = 0
OP_DECODE = 1
OP_PREFILL = 2
OP_DECODE_QUERY = 3
OP_DECODE_ATTENTION = 4
OP_DECODE_OUTPUT = 5
OP_DECODE_MERGED = 6
OP_MHA_DECODE = 7
OP_ATTENTION_BACKWARD = 8

LAYOUT_ROWS = 0
LAYOUT_TILES = 1

c_int, c_size_t, c_void_p, c_float, c_double = (ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p,
                                                ctypes.c_float, ctypes.c_double)


class Config(ctypes.Structure):
    _fields_ = [("d", c_int), ("n_h", c_int), ("d_h", c_int), ("d_c", c_int), ("d_cq", c_int),
                ("d_r", c_int), ("page_size", c_int), ("dtype", c_int),
                ("softmax_scale", c_float), ("rope_base", c_double)]


WEIGHT_ORDER = ("W_DKV", "W_KR", "W_DQ", "W_UQ", "W_QR", "W_UK", "W_UV", "W_O")


class Weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in WEIGHT_ORDER] + [("layout", c_int)]


class MergedWeights(ctypes.Structure):
    _fields_ = [("W_DQ", c_void_p), ("W_QR", c_void_p), ("W_UQK", c_void_p), ("W_OUV", c_void_p),
                ("layout", c_int)]


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None

_P = c_void_p
_SIGS = {
    "mla_status_string": (ctypes.c_char_p, [c_int]),
    "mla_version": (c_int, []),
    "mla_rope_table_init": (c_int, [_P, c_int, _P, _P]),
    "mla_workspace_size": (c_size_t, [_P, c_int, c_int, c_int, c_int]),
    "mla_packed_weights_size": (c_size_t, [_P]),
    "mla_pack_weights": (c_int, [_P, _P, _P, c_size_t, _P, _P]),
    "mla_append_kv": (c_int, [_P, _P, _P, _P, _P, c_int, _P, c_int, _P, c_int, _P, c_size_t, _P]),
    "mla_decode": (c_int, [_P, _P, _P, _P, _P, c_int, _P, c_int, _P, c_int, c_int, _P, c_int,
                           c_int, _P, c_size_t, _P, _P]),
    "mla_decode_noalloc": (c_int, [_P, _P, _P, _P, _P, c_int, _P, c_int, _P, c_int, c_int, _P,
                                   c_int, c_int, _P, _P]),
    "mla_decode_query": (c_int, [_P, _P, _P, _P, c_int, _P, c_int, _P, c_size_t, _P, _P]),
    "mla_decode_attention": (c_int, [_P, _P, _P, c_int, _P, c_int, _P, c_int, c_int, c_int, _P,
                                     c_size_t, _P, _P]),
    "mla_decode_output": (c_int, [_P, _P, _P, c_int, _P, c_size_t, _P, _P]),
    "mla_merge_weights": (c_int, [_P, _P, c_int, _P, _P, _P]),
    "mla_decode_merged": (c_int, [_P, _P, _P, _P, _P, c_int, _P, c_int, _P, c_int, c_int, _P,
                                  c_int, c_int, _P, c_size_t, _P, _P]),
    "mla_mha_decode_attention": (c_int, [_P, _P, _P, c_int, _P, c_int, _P, c_int, c_int, c_float,
                                         c_int, _P, c_size_t, _P, _P]),
    "mla_attention_backward": (c_int, [_P, _P, _P, _P, _P, c_int, _P, c_int, c_int, c_int, _P,
                                       _P, c_size_t, _P, _P, _P, _P, _P]),
    "mla_profile_enable": (c_int, [c_int]),
    "mla_profile_attention_ms": (c_int, [ctypes.POINTER(c_double), ctypes.POINTER(c_int)]),
    "mla_profile_read": (c_int, [ctypes.POINTER(c_double), ctypes.POINTER(c_double),
                                 ctypes.POINTER(c_int)]),
    "mla_prefill": (c_int, [_P, _P, _P, _P, _P, c_int, _P, c_int, c_int, c_int, _P, c_int, _P,
                            c_size_t, _P, _P]),
}


def load() -> ctypes.CDLL:
    """Load libmla.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              f"`python -m mla_latent_kv_15_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().mla_status_string(status).decode()


def _check(fn: str, status: int):
    if status != MLA_OK:
        raise MLAError(fn, status)


# ---------------------------------------------------------------------------
# helpers (torch only for pointers and streams)
# ---------------------------------------------------------------------------

def make_config(shape, page_size: int = 64, dtype: str = "bf16", softmax_scale: float = 0.0,
                rope_base: float = 10000.0) -> Config:
    return Config(shape.d, shape.n_h, shape.d_h, shape.d_c, shape.d_cq, shape.d_r, page_size,
                  MLA_BF16 if dtype == "bf16" else MLA_F32, softmax_scale, rope_base)


def make_weights(tensors: dict) -> Weights:
    """Row-major weights (MLA_LAYOUT_ROWS) from device tensors."""
    return Weights(*[tensors[n].data_ptr() if tensors.get(n) is not None else None
                     for n in WEIGHT_ORDER], LAYOUT_ROWS)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ws(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())


def workspace_size(cfg: Config, op: int, batch: int, max_kv_len: int = 0,
                   num_splits: int = 0) -> int:
    return int(load().mla_workspace_size(ctypes.byref(cfg), op, batch, max_kv_len, num_splits))


def packed_weights_size(cfg: Config) -> int:
    return int(load().mla_packed_weights_size(ctypes.byref(cfg)))


def pack_weights(cfg: Config, weights: Weights, dst, stream=None) -> Weights:
    """Tiled copies (MLA_LAYOUT_TILES) of row-major `weights` in the device
    buffer `dst` (at least packed_weights_size bytes, kept alive by the
    caller while the result is in use)."""
    out = Weights()
    _check("mla_pack_weights", load().mla_pack_weights(
        ctypes.byref(cfg), ctypes.byref(weights), _ptr(dst), dst.numel() * dst.element_size(),
        ctypes.byref(out), _stream(stream)))
    return out


def rope_table_init(cfg: Config, max_pos: int, table, stream=None):
    _check("mla_rope_table_init",
           load().mla_rope_table_init(ctypes.byref(cfg), max_pos, _ptr(table), _stream(stream)))


def append_kv(cfg, weights, h, positions, slot_mapping, rope_table, kv_cache, workspace,
              stream=None):
    wp, wn = _ws(workspace)
    T = h.shape[0]
    _check("mla_append_kv", load().mla_append_kv(
        ctypes.byref(cfg), ctypes.byref(weights), _ptr(h), _ptr(positions), _ptr(slot_mapping), T,
        _ptr(rope_table), rope_table.shape[0], _ptr(kv_cache), kv_cache.shape[0], wp, wn,
        _stream(stream)))


def decode(cfg, weights, h, positions, kv_cache, page_table, kv_lens, max_kv_len, rope_table,
           num_splits, workspace, out, stream=None):
    wp, wn = _ws(workspace)
    _check("mla_decode", load().mla_decode(
        ctypes.byref(cfg), ctypes.byref(weights), _ptr(h), _ptr(positions), _ptr(kv_cache),
        kv_cache.shape[0], _ptr(page_table), page_table.shape[1], _ptr(kv_lens), h.shape[0],
        max_kv_len, _ptr(rope_table), rope_table.shape[0], num_splits, wp, wn, _ptr(out),
        _stream(stream)))


def decode_noalloc(cfg, weights, h, positions, kv_cache, page_table, kv_lens, max_kv_len,
                   rope_table, num_splits, out, stream=None):
    """mla_decode with the library's fixed device scratch array (no workspace)."""
    _check("mla_decode_noalloc", load().mla_decode_noalloc(
        ctypes.byref(cfg), ctypes.byref(weights), _ptr(h), _ptr(positions), _ptr(kv_cache),
        kv_cache.shape[0], _ptr(page_table), page_table.shape[1], _ptr(kv_lens), h.shape[0],
        max_kv_len, _ptr(rope_table), rope_table.shape[0], num_splits, _ptr(out),
        _stream(stream)))


def decode_query(cfg, weights, h, positions, rope_table, workspace, q_abs, stream=None):
    wp, wn = _ws(workspace)
    _check("mla_decode_query", load().mla_decode_query(
        ctypes.byref(cfg), ctypes.byref(weights), _ptr(h), _ptr(positions), h.shape[0],
        _ptr(rope_table), rope_table.shape[0], wp, wn, _ptr(q_abs), _stream(stream)))


def decode_attention(cfg, q_abs, kv_cache, page_table, kv_lens, max_kv_len, num_splits,
                     workspace, latent_out, stream=None):
    wp, wn = _ws(workspace)
    _check("mla_decode_attention", load().mla_decode_attention(
        ctypes.byref(cfg), _ptr(q_abs), _ptr(kv_cache), kv_cache.shape[0], _ptr(page_table),
        page_table.shape[1], _ptr(kv_lens), q_abs.shape[0], max_kv_len, num_splits, wp, wn,
        _ptr(latent_out), _stream(stream)))


def decode_output(cfg, weights, latent_out, workspace, out, stream=None):
    wp, wn = _ws(workspace)
    _check("mla_decode_output", load().mla_decode_output(
        ctypes.byref(cfg), ctypes.byref(weights), _ptr(latent_out), latent_out.shape[0], wp, wn,
        _ptr(out), _stream(stream)))


def prefill(cfg, weights, h, positions, kv_cache, page_table, kv_len, rope_table, workspace, out,
            stream=None):
    wp, wn = _ws(workspace)
    _check("mla_prefill", load().mla_prefill(
        ctypes.byref(cfg), ctypes.byref(weights), _ptr(h), _ptr(positions), _ptr(kv_cache),
        kv_cache.shape[0], _ptr(page_table), page_table.shape[0], kv_len, h.shape[0],
        _ptr(rope_table), rope_table.shape[0], wp, wn, _ptr(out), _stream(stream)))


def merge_weights(cfg, weights: Weights, layout: int, W_UQK, W_OUV, stream=None):
    """W_UQK [n_h*d_c][d_cq] and W_OUV [d][n_h*d_c] from row-major `weights`,
    written in `layout` into the device tensors W_UQK and W_OUV."""
    _check("mla_merge_weights", load().mla_merge_weights(
        ctypes.byref(cfg), ctypes.byref(weights), layout, _ptr(W_UQK), _ptr(W_OUV),
        _stream(stream)))


def decode_merged(cfg, mweights: MergedWeights, h, positions, kv_cache, page_table, kv_lens,
                  max_kv_len, rope_table, num_splits, workspace, out, stream=None):
    wp, wn = _ws(workspace)
    _check("mla_decode_merged", load().mla_decode_merged(
        ctypes.byref(cfg), ctypes.byref(mweights), _ptr(h), _ptr(positions), _ptr(kv_cache),
        kv_cache.shape[0], _ptr(page_table), page_table.shape[1], _ptr(kv_lens), h.shape[0],
        max_kv_len, _ptr(rope_table), rope_table.shape[0], num_splits, wp, wn, _ptr(out),
        _stream(stream)))


def mha_decode_attention(cfg, q, kv_cache, page_table, kv_lens, max_kv_len, num_splits,
                         workspace, out, scale: float = 0.0, stream=None):
    """Baseline: decode attention over an MHA-equivalent cache
    [pages][page][2][n_h][d_h]; q, out [B][n_h][d_h]."""
    wp, wn = _ws(workspace)
    _check("mla_mha_decode_attention", load().mla_mha_decode_attention(
        ctypes.byref(cfg), _ptr(q), _ptr(kv_cache), kv_cache.shape[0], _ptr(page_table),
        page_table.shape[1], _ptr(kv_lens), q.shape[0], max_kv_len, scale, num_splits, wp, wn,
        _ptr(out), _stream(stream)))


def attention_backward(cfg, weights, q, positions, kv_cache, page_table_row, kv_len, dO, workspace,
                       dW_UK, dW_UV, dq, dC, stream=None):
    """Order-A attention backward: gradients of W_UK, W_UV, q and the cached
    rows for one sequence (page_table_row [max_pages]); all fp32 device tensors."""
    wp, wn = _ws(workspace)
    _check("mla_attention_backward", load().mla_attention_backward(
        ctypes.byref(cfg), ctypes.byref(weights), _ptr(q), _ptr(positions), _ptr(kv_cache),
        kv_cache.shape[0], _ptr(page_table_row), page_table_row.shape[0], kv_len, q.shape[0],
        _ptr(dO), wp, wn, _ptr(dW_UK), _ptr(dW_UV), _ptr(dq), _ptr(dC), _stream(stream)))


def profile_enable(on: bool):
    _check("mla_profile_enable", load().mla_profile_enable(1 if on else 0))


def profile_read():
    """(summed attention-kernel ms, summed attention + merge ms, launches)
    since the last read."""
    a, m = c_double(0.0), c_double(0.0)
    n = c_int(0)
    _check("mla_profile_read", load().mla_profile_read(ctypes.byref(a), ctypes.byref(m),
                                                         ctypes.byref(n)))
    return a.value, m.value, n.value


def profile_attention_ms():
    """(summed attention-kernel milliseconds, launches) since the last read."""
    ms = c_double(0.0)
    n = c_int(0)
    _check("mla_profile_attention_ms", load().mla_profile_attention_ms(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
