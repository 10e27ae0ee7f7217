"""Order-A attention backward (mla_attention_backward) against the fp64
oracle's gradients (which are pinned to PyTorch autograd and to finite
differences on the CPU): a small fp32 layer, tiled against row-major weights
(bit for bit), the V2 head shape from a bf16 cache, and the NaN rule for an
invalid query position.
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_15_amd import device, inputs, lib
from tests.gpu_helpers import Layer, cache_from_rows, log, require_lib
from tests.test_gpu_tiles import SMALL, _bits, _pack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


def _bf16_values(a):
    """fp32 numbers that bf16 holds exactly (round to nearest even)."""
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


def _setup(layer, N, T, cid):
    s = layer.shape
    paged = inputs.make_paged([N], layer.page, cid, shuffle=True)
    rows = inputs.make_cache_rows(N, s, cid, layer.dtype)
    cache = cache_from_rows(layer, rows, paged, np.array([0]))
    q = inputs.normal((T, s.n_h, s.d_h + s.d_r), 1.0, cid, inputs.STREAM_QUERY)
    dO = inputs.normal((T, s.n_h, s.d_h), 1.0, cid, inputs.STREAM_QUERY, 1)
    if layer.dtype == "bf16":
        # the bf16 path rounds q and dO to bf16 on entry (a bf16 training step
        # hands them over in bf16): both sides take the same bf16 values
        q, dO = _bf16_values(q), _bf16_values(dO)
    return paged, rows, cache, q, dO


def _run(layer, wts, q, positions, cache, paged, N, dO):
    s = layer.shape
    T = q.shape[0]
    ws = device.workspace(lib.workspace_size(layer.cfg, lib.OP_ATTENTION_BACKWARD, T, N, 0))
    f = lambda *shape: torch.empty(*shape, dtype=torch.float32, device="cuda")  # noqa: E731
    out = dict(dW_UK=f(s.n_h * s.d_h, s.d_c), dW_UV=f(s.n_h * s.d_h, s.d_c),
               dq=f(T, s.n_h, s.d_h + s.d_r), dC=f(N, s.row))
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()  # noqa: E731
    old, layer.wts = layer.wts, wts
    try:
        lib.attention_backward(layer.cfg, layer.wts, torch.from_numpy(q).cuda(), i32(positions),
                               cache, i32(paged.page_table[0]), N, torch.from_numpy(dO).cuda(),
                               ws, out["dW_UK"], out["dW_UV"], out["dq"], out["dC"])
    finally:
        layer.wts = old
    torch.cuda.synchronize()
    return out


def _reference(layer, q, positions, rows, dO):
    s = layer.shape
    W = layer.W64
    r = rows.f64()
    sc = oracle.default_scale(s.d_h, s.d_r)
    g = oracle.attend_order_a_backward(q[:, :, :s.d_h], q[:, :, s.d_h:], positions, r[:, :s.d_c],
                                       r[:, s.d_c:], W["W_UK"], W["W_UV"], sc, dO)
    return dict(dW_UK=g["dW_UK"], dW_UV=g["dW_UV"],
                dq=np.concatenate([g["dq_c"], g["dq_r"]], axis=2),
                dC=np.concatenate([g["dc"], g["dk_r"]], axis=1))


# The output vectors of the error measure: a row of dW_UK or dW_UV (one head
# dimension over the latent), one query token's gradient over all heads
# ([n_h][d_h + d_r]: the token's query vector), and one cached row of dC.  A
# single head's slice of dq can nearly cancel (at one query over two keys,
# dS ~ p_0 p_1 (dP_0 - dP_1) with dO . v_0 close to dO . v_1); measured against
# that slice's own largest entry, bf16 dP resolves it no better than 2^-9 of
# |dP|, so the slice is no vector of its own.
def _vectors(k, v):
    return v.reshape(v.shape[0], -1) if k == "dq" else v.reshape(-1, v.shape[-1])


def _compare(out, ref, tol):
    worst = {}
    for k, v in ref.items():
        got = device.to_f64(out[k]).reshape(v.shape)
        worst[k] = oracle.max_rel_error(_vectors(k, got), _vectors(k, v))
        assert worst[k] < tol, (k, worst[k])
    return worst


def test_small_backward_fp32_and_tiles():
    layer = Layer(SMALL, 51, "f32", page=8)
    N, T = 21, 6
    positions = np.array([0, 5, 20, 13, 19, 7], np.int32)
    paged, rows, cache, q, dO = _setup(layer, N, T, 51)
    log("small backward fp32")
    out = _run(layer, layer.wts, q, positions, cache, paged, N, dO)
    w = _compare(out, _reference(layer, q.astype(np.float64), positions, rows, dO), 1e-4)
    log(f"small backward worst rel err {max(w.values()):.2e}")
    # tiled weights: the same arithmetic from other addresses
    _buf, wt = _pack(layer)
    out_t = _run(layer, wt, q, positions, cache, paged, N, dO)
    for k in out:
        assert np.array_equal(_bits(out[k]), _bits(out_t[k])), k


# The V2 head shape runs on bf16 MFMA: k, v, the scaled q, the softmax
# numerators and the latent gradients dk^C, dv are rounded to bf16 (8
# significant bits) before the products that take them, with fp32 sums; 2e-2
# of each output vector's largest entry is the bf16 bar.  (Rounding an fp32
# dO as well costs up to 2.3e-2 on dW_UV at T = 8, where a row of dW_UV is a
# sum of eight rank-one terms that can nearly cancel, hence bf16-valued q and
# dO on both sides.)
V2_TOL = 2e-2


def test_v2_heads_backward():
    layer = Layer(inputs.V2, 52, "bf16")
    N, T = 96, 8
    positions = np.array([95, 94, 90, 64, 63, 40, 1, 0], np.int32)
    paged, rows, cache, q, dO = _setup(layer, N, T, 52)
    log("v2 backward")
    out = _run(layer, layer.wts, q, positions, cache, paged, N, dO)
    w = _compare(out, _reference(layer, q.astype(np.float64), positions, rows, dO), V2_TOL)
    log(f"v2 backward worst rel err {max(w.values()):.2e}")


def test_v2_backward_ragged_and_tiles():
    """Several query and key blocks with ragged tails (T = 150 of blocks of
    32 and 128, N = 300 of blocks of 128), scattered positions with repeats
    and both ends of the cache; then the tiled weights, bit for bit."""
    layer = Layer(inputs.V2, 54, "bf16")
    N, T = 300, 150
    positions = np.random.default_rng(54).integers(0, N, T).astype(np.int32)
    positions[:5] = [0, N - 1, 127, 128, N - 1]
    paged, rows, cache, q, dO = _setup(layer, N, T, 54)
    log(f"v2 backward T={T} N={N}")
    out = _run(layer, layer.wts, q, positions, cache, paged, N, dO)
    w = _compare(out, _reference(layer, q.astype(np.float64), positions, rows, dO), V2_TOL)
    log(f"v2 backward ragged worst rel err {max(w.values()):.2e}")
    _buf, wt = _pack(layer)
    out_t = _run(layer, wt, q, positions, cache, paged, N, dO)
    for k in out:
        assert np.array_equal(_bits(out[k]), _bits(out_t[k])), k


def test_v2_backward_invalid_position_gives_nan():
    layer = Layer(inputs.V2, 55, "bf16")
    N, T = 70, 40
    positions = np.random.default_rng(55).integers(0, N, T).astype(np.int32)
    positions[5] = N + 3                          # past kv_len
    paged, rows, cache, q, dO = _setup(layer, N, T, 55)
    log("v2 backward invalid position")
    out = _run(layer, layer.wts, q, positions, cache, paged, N, dO)
    dq = device.to_f64(out["dq"])
    for k in ("dW_UK", "dW_UV", "dC"):             # every key sees the bad query
        assert np.isnan(device.to_f64(out[k])).all(), k
    assert np.isnan(dq[5]).all()
    assert np.isfinite(np.delete(dq, 5, axis=0)).all()


def test_backward_invalid_position_gives_nan():
    layer = Layer(SMALL, 53, "f32", page=8)
    N, T = 12, 3
    positions = np.array([4, 12, 7], np.int32)    # 12 is past kv_len
    paged, rows, cache, q, dO = _setup(layer, N, T, 53)
    out = _run(layer, layer.wts, q, positions, cache, paged, N, dO)
    assert np.isnan(device.to_f64(out["dW_UK"])).all()
    assert np.isnan(device.to_f64(out["dW_UV"])).all()
    assert np.isnan(device.to_f64(out["dq"])[1]).all()
