"""Helpers for the GPU tests: seeded layers on the device and the C-ABI calls."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

from mla_latent_kv_15_amd import device, inputs, lib

BASE = 10000.0
TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def require_lib():
    if not os.path.exists(lib.LIB_PATH):
        raise RuntimeError("libmla.so is not built; run __graft_entry__.build() first")
    lib.load()


class Layer:
    """One seeded MLA layer: host weights (exact fp64 copies) and device weights."""

    def __init__(self, shape: inputs.Shape, cid: int, dtype: str, page: int = 64,
                 zero=(), keep_host=True):
        self.shape, self.dtype, self.page = shape, dtype, page
        W = inputs.make_weights(shape, cid, dtype)
        for name in zero:
            W[name] = inputs.Array(np.zeros(W[name].shape, np.float32), dtype)
        self.Wd = device.weights(W)
        self.W64 = {k: v.f64() for k, v in W.items()} if keep_host else None
        self.cfg = lib.make_config(shape, page, dtype, 0.0, BASE)
        self.wts = lib.make_weights(self.Wd)
        self.tdtype = device.storage_dtype(dtype)
        self._rope = None

    def rope(self, max_pos: int) -> torch.Tensor:
        if self._rope is None or self._rope.shape[0] < max_pos:
            t = torch.empty(max_pos, self.shape.d_r // 2, 2, dtype=torch.float32, device="cuda")
            lib.rope_table_init(self.cfg, max_pos, t)
            self._rope = t
        return self._rope

    def empty_cache(self, num_pages: int, fill=float("nan")) -> torch.Tensor:
        return torch.full((num_pages, self.page, self.shape.row), fill, dtype=self.tdtype,
                          device="cuda")

    # -- C-ABI calls ------------------------------------------------------
    def append(self, h: torch.Tensor, positions: np.ndarray, slots: np.ndarray, cache, rope):
        T = h.shape[0]
        ws = device.workspace(lib.workspace_size(self.cfg, lib.OP_APPEND, T))
        pos = torch.from_numpy(np.asarray(positions, np.int32)).cuda()
        sl = torch.from_numpy(np.asarray(slots, np.int32)).cuda()
        lib.append_kv(self.cfg, self.wts, h, pos, sl, rope, cache, ws)

    def decode(self, h, positions, cache, page_table, kv_lens, max_kv_len, rope, num_splits=0):
        B = h.shape[0]
        ws = device.workspace(lib.workspace_size(self.cfg, lib.OP_DECODE, B, max_kv_len, num_splits))
        out = torch.empty(B, self.shape.d, dtype=self.tdtype, device="cuda")
        lib.decode(self.cfg, self.wts, h, _i32(positions), cache, _i32(page_table), _i32(kv_lens),
                   max_kv_len, rope, num_splits, ws, out)
        return out

    def decode_query(self, h, positions, rope):
        B = h.shape[0]
        ws = device.workspace(lib.workspace_size(self.cfg, lib.OP_DECODE_QUERY, B))
        q = torch.empty(B, self.shape.n_h, self.shape.row, dtype=self.tdtype, device="cuda")
        lib.decode_query(self.cfg, self.wts, h, _i32(positions), rope, ws, q)
        return q

    def decode_attention(self, q_abs, cache, page_table, kv_lens, max_kv_len, num_splits=0):
        B = q_abs.shape[0]
        ws = device.workspace(lib.workspace_size(self.cfg, lib.OP_DECODE_ATTENTION, B, max_kv_len,
                                                 num_splits))
        lat = torch.empty(B, self.shape.n_h, self.shape.d_c, dtype=self.tdtype, device="cuda")
        lib.decode_attention(self.cfg, q_abs, cache, _i32(page_table), _i32(kv_lens), max_kv_len,
                             num_splits, ws, lat)
        return lat

    def decode_output(self, lat):
        B = lat.shape[0]
        ws = device.workspace(lib.workspace_size(self.cfg, lib.OP_DECODE_OUTPUT, B))
        out = torch.empty(B, self.shape.d, dtype=self.tdtype, device="cuda")
        lib.decode_output(self.cfg, self.wts, lat, ws, out)
        return out

    def prefill(self, h, positions, cache, page_table_row, kv_len, rope):
        T = h.shape[0]
        ws = device.workspace(lib.workspace_size(self.cfg, lib.OP_PREFILL, T, kv_len))
        out = torch.empty(T, self.shape.d, dtype=self.tdtype, device="cuda")
        lib.prefill(self.cfg, self.wts, h, _i32(positions), cache, _i32(page_table_row), kv_len,
                    rope, ws, out)
        return out


def _i32(a):
    if isinstance(a, torch.Tensor):
        return a
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()


def cache_from_rows(layer: Layer, rows: inputs.Array, paged: inputs.Paged, offsets) -> torch.Tensor:
    """Device cache holding ``rows`` at the slots ``paged`` assigns (NaN elsewhere)."""
    if rows.dtype == "bf16":
        host = inputs.scatter_rows(rows.bits, paged, offsets, fill=0x7FC0)
        return device.bits_tensor(host)
    host = inputs.scatter_rows(rows.f32, paged, offsets, fill=np.float32(np.nan))
    return torch.from_numpy(host).cuda()
