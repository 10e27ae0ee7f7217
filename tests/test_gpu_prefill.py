"""Causal prefill (mla_prefill, order A) on the DeepSeek-V2 head shape, where
the attention runs on bf16 MFMA (one wave per block of 32 queries and head):
query positions in any order with repeats, a context of 300 rows (not a
multiple of the 32-key block), 66 queries (a ragged last block), queries at
positions 0 and N - 1, and a position outside the context (NaN row).  Rows
against the fp64 oracle (a sample) and against mla_decode at kv_len = p + 1
(all rows).
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_15_amd import device, inputs
from tests.gpu_helpers import BASE, TOL, Layer, log, require_lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


def test_v2_prefill_scattered_positions():
    s = inputs.V2
    layer = Layer(s, 71, "bf16")
    N = 300
    H = inputs.make_hidden(N, s, 71, "bf16")
    paged = inputs.make_paged([N], 64, 71, shuffle=True)
    rope = layer.rope(N + 16)
    cache = layer.empty_cache(paged.num_pages)
    h_all = device.tensor(H)
    log("v2 prefill, scattered positions: append 300 rows")
    layer.append(h_all, np.arange(N), paged.slots(0), cache, rope)
    rng = np.random.default_rng(71)
    src = np.concatenate([[0, N - 1, 31, 32, 33, 31], rng.integers(0, N, 59), [7]])
    pos = src.copy()
    pos[-1] = N + 5   # outside the context
    hq = h_all[torch.from_numpy(src).cuda()]
    log("v2 prefill, scattered positions: prefill of 66 queries")
    u = device.to_f64(layer.prefill(hq, pos, cache, paged.page_table[0], N, rope))
    assert np.isnan(u[-1]).all()
    assert np.isfinite(u[:-1]).all()
    # every valid row against decode of the same token at kv_len = p + 1
    P = pos[:-1]
    dec = device.to_f64(layer.decode(hq[:-1], P, cache, np.repeat(paged.page_table, len(P), 0),
                                     P + 1, int(P.max()) + 1, rope))
    xerr = oracle.max_rel_error(u[:-1], dec)
    log(f"prefill vs decode: {xerr:.3e}")
    assert xerr < 2 * TOL["bf16"]
    # a sample against the fp64 oracle
    H64 = H.f64()
    c, kr = oracle.latent_rows(H64, layer.W64["W_DKV"], layer.W64["W_KR"], np.arange(N), BASE)
    sel = [0, 1, 2, 3, 7, 20, 64]
    ref = oracle.prefill_order_a(H64[src], pos, c, kr, layer.W64, s.n_h, BASE, rows=sel)
    err = oracle.max_rel_error(u[sel], ref)
    log(f"prefill vs oracle: {err:.3e}")
    assert err < TOL["bf16"]
