"""Causal prefill (mla_prefill, order A) on the DeepSeek-V2 head shape, where
the attention runs on bf16 MFMA (one wave per block of 32 queries and head):
query positions in any order with repeats, a context of 300 rows (not a
multiple of the 32-key block), 66 or 147 queries (a ragged last block), queries at
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


@pytest.mark.parametrize("n_rand", [59, 140])
def test_v2_prefill_scattered_positions(n_rand):
    """66 queries take the weight-streaming products (RoPE query input in
    fp32, then rotated); 147 the tiled ones, RoPE in the product's epilogue."""
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
    src = np.concatenate([[0, N - 1, 31, 32, 33, 31], rng.integers(0, N, n_rand), [7]])
    pos = src.copy()
    pos[-1] = N + 5   # outside the context
    hq = h_all[torch.from_numpy(src).cuda()]
    log(f"v2 prefill, scattered positions: prefill of {len(src)} queries")
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


def test_v2_prefill_score_jumps():
    """Hidden rows scaled by 6 at positions 40, 130 and 250: their keys lift
    the score maximum of many (query, head) pairs by far more than 8 log2
    units in blocks after the first, so the prefill's softmax reference moves
    (and O is rescaled) mid-stream, not only at a query's first key block.
    That the data does so is checked on the CPU from the oracle's scores;
    rows after each jump against the fp64 oracle, the last 64 against decode."""
    s = inputs.V2
    layer = Layer(s, 72, "bf16")
    N = 300
    jumps = [40, 130, 250]
    f = inputs.normal((N, s.d), 1.0, 72, inputs.STREAM_HIDDEN)
    f[jumps] *= 6.0   # (larger factors make the bf16 rounding of the scores dominate)
    H = inputs.Array(f, "bf16")
    H64 = H.f64()
    W = layer.W64
    c, kr = oracle.latent_rows(H64, W["W_DKV"], W["W_KR"], np.arange(N), BASE)
    # the data's own jumps: running maximum (log2 units) over 32-key blocks
    scale = oracle.default_scale(s.d_h, s.d_r) / np.log(2.0)
    t = N - 1
    q_c, q_r = oracle.query(H64[t], W["W_DQ"], W["W_UQ"], W["W_QR"], t, s.n_h, BASE)
    lifted = 0
    for i in range(s.n_h):
        k = np.concatenate([c @ W["W_UK"][i * s.d_h:(i + 1) * s.d_h].T, kr], axis=1)
        sc = k @ np.concatenate([q_c[i], q_r[i]]) * scale
        run = np.maximum.accumulate([sc[j0:j0 + 32].max() for j0 in range(0, N, 32)])
        lifted += int((np.diff(run) > 8.0).any())
    log(f"prefill score jumps: {lifted} of {s.n_h} heads of query {t} lift their maximum by > 8")
    assert lifted >= 8
    paged = inputs.make_paged([N], 64, 72, shuffle=True)
    rope = layer.rope(N + 16)
    cache = layer.empty_cache(paged.num_pages)
    h_all = device.tensor(H)
    layer.append(h_all, np.arange(N), paged.slots(0), cache, rope)
    pos = np.arange(N)
    u = device.to_f64(layer.prefill(h_all, pos, cache, paged.page_table[0], N, rope))
    assert np.isfinite(u).all()
    P = np.arange(N - 64, N)
    dec = device.to_f64(layer.decode(h_all[N - 64:], P, cache, np.repeat(paged.page_table, 64, 0),
                                     P + 1, N, rope))
    xerr = oracle.max_rel_error(u[N - 64:], dec)
    log(f"prefill vs decode (jumps): {xerr:.3e}")
    assert xerr < 2 * TOL["bf16"]
    sel = [0, 39, 40, 41, 100, 129, 130, 131, 249, 250, 251, 299]
    ref = oracle.prefill_order_a(H64, pos, c, kr, W, s.n_h, BASE, rows=sel)
    err = oracle.max_rel_error(u[sel], ref)
    log(f"prefill vs oracle (jumps): {err:.3e}")
    assert err < TOL["bf16"]
