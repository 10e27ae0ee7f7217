"""Seeded synthetic inputs shared by the GPU path, the tests and the bench.

This module only draws random numbers and changes their storage format
(float32 -> bfloat16 bit patterns, page tables, length mixes).  It holds none
of the attention arithmetic, so the oracle and the HIP library can both be fed
from it without sharing any of the method's code.

Distributions follow the layer the pages describe (DeepSeek-V2 shapes):
hidden states ~ N(0, 1); every weight ``W[out][in]`` ~ N(0, 1/in); cached
latent rows ~ N(0, 1), which is the distribution ``W_DKV h`` has under those
weights.  Seeds come from ``numpy.random.SeedSequence([config_id, stream])``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np

# stream ids inside one config's SeedSequence
STREAM_WEIGHTS = 0
STREAM_HIDDEN = 1
STREAM_LENGTHS = 2
STREAM_PAGES = 3
STREAM_CACHE = 4
STREAM_QUERY = 5


@dataclasses.dataclass(frozen=True)
class Shape:
    d: int      # model dim
    n_h: int    # heads
    d_h: int    # per-head dim (content part)
    d_c: int    # KV latent dim
    d_cq: int   # query latent dim
    d_r: int    # decoupled RoPE dim

    @property
    def row(self) -> int:
        """Numbers cached per token: latent plus shared RoPE key."""
        return self.d_c + self.d_r


# DeepSeek-V2 layer shape and the tiny fp32 layer
V2 = Shape(d=5120, n_h=128, d_h=128, d_c=512, d_cq=1536, d_r=64)
TINY = Shape(d=64, n_h=4, d_h=16, d_c=32, d_cq=48, d_r=8)

WEIGHT_NAMES = ("W_DKV", "W_KR", "W_DQ", "W_UQ", "W_QR", "W_UK", "W_UV", "W_O")


def weight_shapes(s: Shape) -> Dict[str, tuple]:
    """Row-major [out][in] shapes, y = W x."""
    return {
        "W_DKV": (s.d_c, s.d),
        "W_KR": (s.d_r, s.d),
        "W_DQ": (s.d_cq, s.d),
        "W_UQ": (s.n_h * s.d_h, s.d_cq),
        "W_QR": (s.n_h * s.d_r, s.d_cq),
        "W_UK": (s.n_h * s.d_h, s.d_c),
        "W_UV": (s.n_h * s.d_h, s.d_c),
        "W_O": (s.d, s.n_h * s.d_h),
    }


def _rng(config_id: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, stream, sub])))


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = np.where(nan, np.uint32(0x7FC0), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Array:
    """A synthetic array in the storage dtype plus its exact float64 widening."""

    def __init__(self, f32: np.ndarray, dtype: str):
        assert dtype in ("bf16", "f32")
        self.dtype = dtype
        if dtype == "bf16":
            self.bits = f32_to_bf16_bits(f32)
            self.f32 = bf16_bits_to_f32(self.bits)
        else:
            self.bits = None
            self.f32 = np.ascontiguousarray(f32, dtype=np.float32)

    @property
    def shape(self):
        return self.f32.shape

    def f64(self) -> np.ndarray:
        return self.f32.astype(np.float64)

    def storage(self) -> np.ndarray:
        """What goes to the device: uint16 bf16 bits or float32."""
        return self.bits if self.dtype == "bf16" else self.f32


def normal(shape, std: float, config_id: int, stream: int, sub: int = 0) -> np.ndarray:
    g = _rng(config_id, stream, sub)
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def make_weights(s: Shape, config_id: int, dtype: str) -> Dict[str, Array]:
    """Every weight W[out][in] ~ N(0, 1/in)."""
    out = {}
    for i, (name, shp) in enumerate(weight_shapes(s).items()):
        out[name] = Array(normal(shp, float(shp[1]) ** -0.5, config_id, STREAM_WEIGHTS, i), dtype)
    return out


def make_hidden(T: int, s: Shape, config_id: int, dtype: str, sub: int = 0) -> Array:
    return Array(normal((T, s.d), 1.0, config_id, STREAM_HIDDEN, sub), dtype)


def make_cache_rows(N: int, s: Shape, config_id: int, dtype: str, sub: int = 0) -> Array:
    """N latent cache rows [c_KV | k_R] ~ N(0, 1)."""
    return Array(normal((N, s.row), 1.0, config_id, STREAM_CACHE, sub), dtype)


def make_lengths(B: int, lo: int, hi: int, config_id: int) -> np.ndarray:
    """Context lengths uniform on the integers [lo, hi]."""
    return _rng(config_id, STREAM_LENGTHS).integers(lo, hi + 1, size=B).astype(np.int32)


@dataclasses.dataclass
class Paged:
    """A paged cache layout for a batch of sequences.

    ``page_table[b][i]`` is the physical page that holds tokens
    [i*page_size, (i+1)*page_size) of sequence b; unused entries are -1.
    """
    kv_lens: np.ndarray      # int32 [B]
    page_table: np.ndarray   # int32 [B][max_pages]
    num_pages: int
    page_size: int

    def slot(self, b: int, t: int) -> int:
        return int(self.page_table[b, t // self.page_size]) * self.page_size + t % self.page_size

    def slots(self, b: int) -> np.ndarray:
        t = np.arange(int(self.kv_lens[b]))
        return self.page_table[b, t // self.page_size].astype(np.int64) * self.page_size + t % self.page_size


def make_paged(kv_lens: np.ndarray, page_size: int, config_id: int, shuffle: bool = True,
               extra_pages: int = 0, max_pages: int | None = None) -> Paged:
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    need = [(int(n) + page_size - 1) // page_size for n in kv_lens]
    total = sum(need) + extra_pages
    mp = max(need) if max_pages is None else max_pages
    perm = np.arange(total, dtype=np.int32)
    if shuffle:
        perm = _rng(config_id, STREAM_PAGES).permutation(total).astype(np.int32)
    pt = np.full((len(kv_lens), max(mp, 1)), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[k:k + n]
        k += n
    return Paged(kv_lens=kv_lens, page_table=pt, num_pages=total, page_size=page_size)


def scatter_rows(rows: np.ndarray, paged: Paged, row_offsets: np.ndarray, fill=0) -> np.ndarray:
    """Place per-sequence rows into a [num_pages][page_size][row] cache array.

    ``rows`` is the concatenation of every sequence's rows; sequence b's rows
    start at ``row_offsets[b]``.  Pure indexing (a storage layout), no arithmetic.
    """
    width = rows.shape[1]
    cache = np.full((paged.num_pages * paged.page_size, width), fill, dtype=rows.dtype)
    for b in range(len(paged.kv_lens)):
        n = int(paged.kv_lens[b])
        cache[paged.slots(b)] = rows[row_offsets[b]:row_offsets[b] + n]
    return cache.reshape(paged.num_pages, paged.page_size, width)
