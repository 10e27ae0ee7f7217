"""Tiled weight layout (MLA_LAYOUT_TILES) on the GPU.

mla_pack_weights is checked element by element against an independent numpy
rearrangement of the row-major matrices.  Every entry point then runs once
with row-major and once with tiled weights: the kernels read the same values
in the same arithmetic order from other addresses, so the results must agree
bit for bit; the tiled decode of the small layer is also checked against the
oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_15_amd import device, inputs, lib
from tests.gpu_helpers import BASE, TOL, Layer, cache_from_rows, log, require_lib

pytestmark = pytest.mark.gpu

# smallest layer whose matrices all admit 16 x 32 tiles (generic kernels)
SMALL = inputs.Shape(d=64, n_h=4, d_h=16, d_c=32, d_cq=64, d_r=16)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


def _tiles_np(W: np.ndarray) -> np.ndarray:
    """[R][C] -> [R/16][C/32][C%32 // 8][R%16][C%8], flattened."""
    R, C = W.shape
    return W.reshape(R // 16, 16, C // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    it = torch.int16 if t.element_size() == 2 else torch.int32
    return t.view(it).numpy()


def _pack(layer: Layer):
    buf = device.workspace(lib.packed_weights_size(layer.cfg))
    wt = lib.pack_weights(layer.cfg, layer.wts, buf)
    torch.cuda.synchronize()
    return buf, wt


class _Tiled:
    """Run a Layer's calls with its packed weights inside the block."""

    def __init__(self, layer, wt):
        self.layer, self.wt = layer, wt

    def __enter__(self):
        self.rows, self.layer.wts = self.layer.wts, self.wt

    def __exit__(self, *exc):
        self.layer.wts = self.rows


@pytest.mark.parametrize("shape,dtype", [(SMALL, "f32"), (SMALL, "bf16"), (inputs.V2, "bf16")])
def test_pack_matches_rearrangement(shape, dtype):
    layer = Layer(shape, 21, dtype, keep_host=False)
    log(f"pack {shape} {dtype}")
    buf, wt = _pack(layer)
    assert wt.layout == lib.LAYOUT_TILES
    raw = buf.view(torch.uint8)
    off = 0
    for name in lib.WEIGHT_ORDER:
        src = layer.Wd[name]
        nbytes = src.numel() * src.element_size()
        assert getattr(wt, name) == buf.data_ptr() + off, name
        got = _bits(raw[off:off + nbytes].view(src.dtype))
        want = _tiles_np(_bits(src).reshape(src.shape))
        assert np.array_equal(got, want), name
        off += (nbytes + 255) // 256 * 256
    assert off == lib.packed_weights_size(layer.cfg)


@pytest.mark.parametrize("B", [64, 130])
def test_v2_decode_tiles_bit_identical(B):
    s = inputs.V2
    layer = Layer(s, 22, "bf16", keep_host=False)
    L = inputs.make_lengths(B, 100, 3000, 22)
    kv = (L + 1).astype(np.int32)
    paged = inputs.make_paged(kv, 64, 22, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(kv)[:-1]]).astype(np.int64)
    rows = inputs.make_cache_rows(int(kv.sum()), s, 22, "bf16")
    cache = cache_from_rows(layer, rows, paged, offs)
    hq = device.tensor(inputs.make_hidden(B, s, 22, "bf16"))
    rope = layer.rope(int(kv.max()) + 1)
    _buf, wt = _pack(layer)
    log(f"v2 decode rows / tiles, B={B}")
    out_r = layer.decode(hq, L, cache, paged.page_table, kv, int(kv.max()), rope)
    q_r = layer.decode_query(hq, L, rope)
    lat = layer.decode_attention(q_r, cache, paged.page_table, kv, int(kv.max()))
    u_r = layer.decode_output(lat)
    with _Tiled(layer, wt):
        out_t = layer.decode(hq, L, cache, paged.page_table, kv, int(kv.max()), rope)
        q_t = layer.decode_query(hq, L, rope)
        u_t = layer.decode_output(lat)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out_r), _bits(out_t))
    assert np.array_equal(_bits(q_r), _bits(q_t))
    assert np.array_equal(_bits(u_r), _bits(u_t))
    assert np.isfinite(device.to_f64(out_t)).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_generic_tiles_bit_identical(dtype):
    s = SMALL
    layer = Layer(s, 23, dtype, page=8)
    N = 21
    H = inputs.make_hidden(N, s, 23, dtype)
    paged = inputs.make_paged([N], 8, 23, shuffle=True)
    rope = layer.rope(64)
    _buf, wt = _pack(layer)
    h = device.tensor(H)
    log(f"small {dtype} append / decode / prefill, rows and tiles")
    caches, outs, pre = [], [], []
    for tiled in (False, True):
        cache = layer.empty_cache(paged.num_pages)
        ctx = _Tiled(layer, wt) if tiled else None
        if ctx:
            ctx.__enter__()
        try:
            layer.append(h, np.arange(N), paged.slots(0), cache, rope)
            outs.append(layer.decode(h[-1:], [N - 1], cache, paged.page_table, [N], N, rope))
            pre.append(layer.prefill(h[-5:], np.arange(N - 5, N), cache, paged.page_table[0], N,
                                     rope))
        finally:
            if ctx:
                ctx.__exit__()
        caches.append(cache)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(caches[0]), _bits(caches[1]))
    assert np.array_equal(_bits(outs[0]), _bits(outs[1]))
    assert np.array_equal(_bits(pre[0]), _bits(pre[1]))
    u = device.to_f64(outs[1])[0]
    ref = oracle.decode_from_hidden(H.f64(), layer.W64, s.n_h, BASE, order="A")
    assert oracle.max_rel_error(u, ref) < TOL[dtype]
