"""Order B on matrices multiplied out ahead of time (mla_merge_weights,
mla_decode_merged) against the fp64 oracle.

The merged matrices are checked against the oracle's products of the same
weights (sampled heads at the V2 shape), the tiled copy against a numpy
rearrangement of the row-major one, and the merged decode against order A.
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_15_amd import device, inputs, lib
from tests.gpu_helpers import BASE, TOL, Layer, cache_from_rows, log, require_lib
from tests.test_gpu_tiles import SMALL, _bits, _pack, _tiles_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


def _merge(layer, layout):
    s = layer.shape
    dt = layer.tdtype
    Mq = torch.empty(s.n_h * s.d_c, s.d_cq, dtype=dt, device="cuda")
    Mo = torch.empty(s.d, s.n_h * s.d_c, dtype=dt, device="cuda")
    lib.merge_weights(layer.cfg, layer.wts, layout, Mq, Mo)
    return Mq, Mo


def _decode_merged(layer, mw, h, positions, cache, page_table, kv_lens, max_kv_len, rope):
    B = h.shape[0]
    ws = device.workspace(lib.workspace_size(layer.cfg, lib.OP_DECODE_MERGED, B, max_kv_len, 0))
    out = torch.empty(B, layer.shape.d, dtype=layer.tdtype, device="cuda")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()  # noqa: E731
    lib.decode_merged(layer.cfg, mw, h, i32(positions), cache, i32(page_table), i32(kv_lens),
                      max_kv_len, rope, 0, ws, out)
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_merge_and_decode(dtype):
    s = SMALL
    layer = Layer(s, 31, dtype, page=8)
    log(f"small merged {dtype}")
    Mq, Mo = _merge(layer, lib.LAYOUT_ROWS)
    Tq, To = _merge(layer, lib.LAYOUT_TILES)
    torch.cuda.synchronize()
    W = layer.W64
    rq = oracle.merged_query_matrix(W["W_UQ"], W["W_UK"], s.n_h)
    ro = oracle.merged_output_matrix(W["W_O"], W["W_UV"], s.n_h)
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert oracle.max_rel_error(device.to_f64(Mq), rq) < tol
    assert oracle.max_rel_error(device.to_f64(Mo), ro) < tol
    assert np.array_equal(_bits(Tq).reshape(-1), _tiles_np(_bits(Mq).reshape(Mq.shape)))
    assert np.array_equal(_bits(To).reshape(-1), _tiles_np(_bits(Mo).reshape(Mo.shape)))
    # decode from the merged matrices, both layouts, against order A
    N = 21
    H = inputs.make_hidden(N, s, 31, dtype)
    paged = inputs.make_paged([N], 8, 31, shuffle=True)
    rope = layer.rope(64)
    cache = layer.empty_cache(paged.num_pages)
    h = device.tensor(H)
    layer.append(h, np.arange(N), paged.slots(0), cache, rope)
    _buf, wt = _pack(layer)
    ref = oracle.decode_from_hidden(H.f64(), W, s.n_h, BASE, order="A")
    for lay, (q, o), dq, qr in ((lib.LAYOUT_ROWS, (Mq, Mo), layer.Wd["W_DQ"], layer.Wd["W_QR"]),
                                (lib.LAYOUT_TILES, (Tq, To), wt.W_DQ, wt.W_QR)):
        mw = lib.MergedWeights(dq if isinstance(dq, int) else dq.data_ptr(),
                               qr if isinstance(qr, int) else qr.data_ptr(),
                               q.data_ptr(), o.data_ptr(), lay)
        out = _decode_merged(layer, mw, h[-1:], [N - 1], cache, paged.page_table, [N], N, rope)
        torch.cuda.synchronize()
        err = oracle.max_rel_error(device.to_f64(out)[0], ref)
        log(f"small merged {dtype} layout {lay}: rel err {err:.2e}")
        assert err < TOL[dtype]


def test_v2_merge_sampled_heads():
    s = inputs.V2
    layer = Layer(s, 32, "bf16")
    log("v2 merge (rows)")
    Mq, Mo = _merge(layer, lib.LAYOUT_ROWS)
    torch.cuda.synchronize()
    W = layer.W64
    for i in (0, 77, 127):
        hq = slice(i * s.d_h, (i + 1) * s.d_h)
        rq = W["W_UK"][hq].T @ W["W_UQ"][hq]
        ro = W["W_O"][:, hq] @ W["W_UV"][hq]
        gq = device.to_f64(Mq[i * s.d_c:(i + 1) * s.d_c])
        go = device.to_f64(Mo[:, i * s.d_c:(i + 1) * s.d_c])
        assert oracle.max_rel_error(gq, rq) < 1e-2
        assert oracle.max_rel_error(go, ro) < 1e-2


def test_v2_decode_merged_batch():
    s = inputs.V2
    layer = Layer(s, 33, "bf16")
    B = 8
    L = inputs.make_lengths(B, 100, 1500, 33)
    kv = (L + 1).astype(np.int32)
    paged = inputs.make_paged(kv, 64, 33, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(kv)[:-1]]).astype(np.int64)
    rows = inputs.make_cache_rows(int(kv.sum()), s, 33, "bf16")
    cache = cache_from_rows(layer, rows, paged, offs)
    Hq = inputs.make_hidden(B, s, 33, "bf16")
    rope = layer.rope(int(kv.max()) + 1)
    _buf, wt = _pack(layer)
    log("v2 merge (tiles)")
    Tq, To = _merge(layer, lib.LAYOUT_TILES)
    mw = lib.MergedWeights(wt.W_DQ, wt.W_QR, Tq.data_ptr(), To.data_ptr(), lib.LAYOUT_TILES)
    out = _decode_merged(layer, mw, device.tensor(Hq), L, cache, paged.page_table, kv,
                         int(kv.max()), rope)
    torch.cuda.synchronize()
    u = device.to_f64(out)
    W = layer.W64
    r64 = rows.f64()
    sc = oracle.default_scale(s.d_h, s.d_r)
    worst = 0.0
    for b in range(B):
        # the unmerged order B of the oracle (equal to order A, see the pins)
        r = r64[offs[b]:offs[b] + kv[b]]
        q_c, q_r = oracle.query(Hq.f64()[b], W["W_DQ"], W["W_UQ"], W["W_QR"], int(L[b]), s.n_h,
                                BASE)
        Qt = oracle.absorbed_query(q_c, q_r, W["W_UK"], sc)
        ref = oracle.latent_output(oracle.latent_attention(Qt, r, s.d_c), W["W_UV"], W["W_O"])
        worst = max(worst, oracle.max_rel_error(u[b], ref))
    log(f"v2 merged decode worst rel err {worst:.3e}")
    assert worst < TOL["bf16"]


def test_v2_decode_merged_many_rows():
    """More than one 64-row activation block: merged and unmerged decode of
    the same batch agree within the bf16 tolerance (each is checked against
    the oracle elsewhere)."""
    s = inputs.V2
    layer = Layer(s, 34, "bf16", keep_host=False)
    B = 70
    L = inputs.make_lengths(B, 50, 600, 34)
    kv = (L + 1).astype(np.int32)
    paged = inputs.make_paged(kv, 64, 34, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(kv)[:-1]]).astype(np.int64)
    rows = inputs.make_cache_rows(int(kv.sum()), s, 34, "bf16")
    cache = cache_from_rows(layer, rows, paged, offs)
    hq = device.tensor(inputs.make_hidden(B, s, 34, "bf16"))
    rope = layer.rope(int(kv.max()) + 1)
    _buf, wt = _pack(layer)
    Tq, To = _merge(layer, lib.LAYOUT_TILES)
    mw = lib.MergedWeights(wt.W_DQ, wt.W_QR, Tq.data_ptr(), To.data_ptr(), lib.LAYOUT_TILES)
    log("v2 merged decode, B=70")
    um = device.to_f64(_decode_merged(layer, mw, hq, L, cache, paged.page_table, kv,
                                      int(kv.max()), rope))
    uu = device.to_f64(layer.decode(hq, L, cache, paged.page_table, kv, int(kv.max()), rope))
    torch.cuda.synchronize()
    assert np.isfinite(um).all()
    assert oracle.max_rel_error(um, uu) < TOL["bf16"]
