"""The MHA-equivalent decode baseline (mla_mha_decode_attention) against the
fp64 oracle's multi-head attention: a small layer in fp32 and bf16, and the
V2 head shape (128 heads of 128) with shuffled pages, forced and automatic
splits, and a sequence with an invalid page id (NaN output).
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_15_amd import device, inputs, lib
from tests.gpu_helpers import TOL, log, require_lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


def _case(n_h, d_h, lens, page, dtype, cid, shuffle=True):
    s = inputs.Shape(d=64, n_h=n_h, d_h=d_h, d_c=32, d_cq=64, d_r=16)
    cfg = lib.make_config(s, page, dtype)
    kv = np.asarray(lens, np.int32)
    paged = inputs.make_paged(kv, page, cid, shuffle=shuffle)
    offs = np.concatenate([[0], np.cumsum(kv)[:-1]]).astype(np.int64)
    width = 2 * n_h * d_h
    rows = inputs.Array(inputs.normal((int(kv.sum()), width), 1.0, cid, inputs.STREAM_CACHE), dtype)
    host = inputs.scatter_rows(rows.storage(), paged, offs, fill=0)
    cache = device.bits_tensor(host) if dtype == "bf16" else torch.from_numpy(host).cuda()
    q = inputs.Array(inputs.normal((len(kv), n_h, d_h), 1.0, cid, inputs.STREAM_QUERY), dtype)
    return cfg, kv, paged, offs, rows, cache, q


def _run(cfg, q, cache, paged, kv, splits, dtype):
    B, n_h, d_h = q.shape
    ws = device.workspace(lib.workspace_size(cfg, lib.OP_MHA_DECODE, B, int(kv.max()), splits))
    out = torch.empty(B, n_h, d_h, dtype=device.storage_dtype(dtype), device="cuda")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()  # noqa: E731
    lib.mha_decode_attention(cfg, device.tensor(q), cache, i32(paged.page_table), i32(kv),
                             int(kv.max()), splits, ws, out)
    torch.cuda.synchronize()
    return device.to_f64(out)


def _check(o, q, rows, kv, offs, n_h, d_h, tol, skip=()):
    sc = 1.0 / np.sqrt(d_h)
    r = rows.f64()
    worst = 0.0
    for b in range(len(kv)):
        if b in skip:
            continue
        blk = r[offs[b]:offs[b] + kv[b]].reshape(kv[b], 2, n_h, d_h)
        ref = oracle.mha_attention(q.f64()[b], blk[:, 0], blk[:, 1], sc)
        worst = max(worst, oracle.max_rel_error(o[b], ref))
    assert worst < tol, worst
    return worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_mha(dtype):
    n_h, d_h = 4, 32
    cfg, kv, paged, offs, rows, cache, q = _case(n_h, d_h, [1, 7, 40, 65], 8, dtype, 41)
    for splits in (0, 3):
        log(f"small mha {dtype} splits={splits}")
        o = _run(cfg, q, cache, paged, kv, splits, dtype)
        _check(o, q, rows, kv, offs, n_h, d_h, TOL[dtype])


def test_v2_heads_mha():
    n_h, d_h = 128, 128
    lens = inputs.make_lengths(3, 100, 900, 42)
    cfg, kv, paged, offs, rows, cache, q = _case(n_h, d_h, lens, 64, "bf16", 42)
    for splits in (0, 2):
        log(f"v2 mha splits={splits}")
        o = _run(cfg, q, cache, paged, kv, splits, "bf16")
        w = _check(o, q, rows, kv, offs, n_h, d_h, TOL["bf16"])
        log(f"v2 mha worst rel err {w:.2e}")
    # an out-of-range page id gives that sequence NaN and leaves the others
    bad = paged.page_table.copy()
    bad[1, 0] = paged.num_pages + 5
    broken = inputs.Paged(kv_lens=paged.kv_lens, page_table=bad, num_pages=paged.num_pages,
                          page_size=paged.page_size)
    o = _run(cfg, q, cache, broken, kv, 0, "bf16")
    assert np.isnan(o[1]).all()
    _check(o, q, rows, kv, offs, n_h, d_h, TOL["bf16"], skip=(1,))
