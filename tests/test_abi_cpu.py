"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

from mla_latent_kv_15_amd import inputs, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        from mla_latent_kv_15_amd import build
        build.build()
    return lib.load()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _header_functions()
    assert "mla_decode" in names and "mla_append_kv" in names and "mla_prefill" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(lib._SIGS)


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.status_string(code) and lib.status_string(code) != "unknown status"
    assert lib.status_string(7) == "unknown status"
    assert L.mla_version() >= 100


def _cfg(shape=inputs.V2, dtype="bf16", page=64):
    return lib.make_config(shape, page, dtype)


def test_workspace_sizes(L):
    c = _cfg()
    assert lib.workspace_size(c, lib.OP_APPEND, 10) == ((10 * 576 * 4 + 255) // 256) * 256
    d1 = lib.workspace_size(c, lib.OP_DECODE, 64, 8193, 0)
    d2 = lib.workspace_size(c, lib.OP_DECODE, 64, 8193, 4)
    assert d1 > 0 and d2 > 0
    assert lib.workspace_size(c, lib.OP_DECODE_QUERY, 1) > 0
    assert lib.workspace_size(c, lib.OP_PREFILL, 4096, 4096) > 4096 * 128 * 192 * 4
    bad = _cfg()
    bad.d_r = 63
    assert lib.workspace_size(bad, lib.OP_DECODE, 1, 1, 0) == 0
    assert lib.workspace_size(c, 99, 1, 1, 0) == 0


def test_invalid_arguments_rejected_before_launch(L):
    c = _cfg()
    w = lib.Weights(*([None] * 8))
    z = ctypes.c_void_p(0)
    # null config / null weights
    assert L.mla_decode(None, None, z, z, z, 1, z, 1, z, 1, 1, z, 1, 0, z, 0, z, z) == lib.MLA_ERR_INVALID_ARG
    assert L.mla_decode(ctypes.byref(c), ctypes.byref(w), z, z, z, 1, z, 1, z, 1, 1, z, 1, 0, z, 0,
                        z, z) == lib.MLA_ERR_INVALID_ARG
    # bad geometry
    for field, val in (("d_r", 7), ("n_h", 0), ("page_size", 0), ("dtype", 5)):
        b = _cfg()
        setattr(b, field, val)
        assert L.mla_rope_table_init(ctypes.byref(b), 10, ctypes.c_void_p(256), None) == lib.MLA_ERR_INVALID_ARG
    assert L.mla_rope_table_init(ctypes.byref(c), 0, ctypes.c_void_p(256), None) == lib.MLA_ERR_INVALID_ARG
    assert L.mla_rope_table_init(ctypes.byref(c), 10, None, None) == lib.MLA_ERR_INVALID_ARG
    # fake non-null device pointers: validation must fail before they are used
    p = ctypes.c_void_p(4096)
    # max_kv_len beyond the page table's reach
    assert L.mla_decode_attention(ctypes.byref(c), p, p, 4, p, 2, p, 1, 129, 0, p, 1 << 30, p,
                                  None) == lib.MLA_ERR_INVALID_ARG
    # negative sizes
    assert L.mla_decode_attention(ctypes.byref(c), p, p, 4, p, 2, p, -1, 10, 0, p, 1 << 30, p,
                                  None) == lib.MLA_ERR_INVALID_ARG
    # workspace too small / misaligned
    assert L.mla_decode_attention(ctypes.byref(c), p, p, 4, p, 2, p, 1, 100, 0, p, 16, p,
                                  None) == lib.MLA_ERR_WORKSPACE
    assert L.mla_decode_attention(ctypes.byref(c), p, p, 4, p, 2, p, 1, 100, 0,
                                  ctypes.c_void_p(4096 + 8), 1 << 40, p, None) == lib.MLA_ERR_WORKSPACE
    # unsupported: a latent too wide for the generic kernels
    u = lib.make_config(inputs.Shape(d=64, n_h=4, d_h=16, d_c=2048, d_cq=48, d_r=8), 64, "f32")
    assert L.mla_decode_attention(ctypes.byref(u), p, p, 4, p, 2, p, 1, 100, 0, p, 1 << 40, p,
                                  None) == lib.MLA_ERR_UNSUPPORTED
    # append: missing weights, zero pages
    assert L.mla_append_kv(ctypes.byref(c), ctypes.byref(w), p, p, p, 3, p, 10, p, 1, p, 1 << 30,
                           None) == lib.MLA_ERR_INVALID_ARG
    wf = lib.Weights(*([4096] * 8))
    assert L.mla_append_kv(ctypes.byref(c), ctypes.byref(wf), p, p, p, 3, p, 10, p, 0, p, 1 << 30,
                           None) == lib.MLA_ERR_INVALID_ARG
    # prefill: kv_len beyond the page table
    assert L.mla_prefill(ctypes.byref(c), ctypes.byref(wf), p, p, p, 8, p, 1, 65, 4, p, 100, p,
                         1 << 40, p, None) == lib.MLA_ERR_INVALID_ARG


def test_empty_batches_are_noops(L):
    c = _cfg()
    wf = lib.Weights(*([4096] * 8))
    z = None
    assert L.mla_append_kv(ctypes.byref(c), ctypes.byref(wf), z, z, z, 0, z, 0, z, 0, z, 0, z) == 0
    assert L.mla_decode_attention(ctypes.byref(c), z, z, 0, z, 0, z, 0, 0, 0, z, 0, z, z) == 0
    assert L.mla_decode_output(ctypes.byref(c), ctypes.byref(wf), z, 0, z, 0, z, z) == 0
    assert L.mla_prefill(ctypes.byref(c), ctypes.byref(wf), z, z, z, 0, z, 0, 0, 0, z, 0, z, 0, z,
                         z) == 0


def test_packed_weights_size_and_checks(L):
    """Tiled weights: byte count, geometry support and argument checks, all
    decided on the host before anything is enqueued."""
    c = _cfg()
    s = inputs.V2
    mats = [s.d_c * s.d, s.d_r * s.d, s.d_cq * s.d, s.n_h * s.d_h * s.d_cq, s.n_h * s.d_r * s.d_cq,
            s.n_h * s.d_h * s.d_c, s.n_h * s.d_h * s.d_c, s.d * s.n_h * s.d_h]
    need = sum(((2 * m + 255) // 256) * 256 for m in mats)
    assert lib.packed_weights_size(c) == need
    assert lib.packed_weights_size(_cfg(dtype="f32")) == sum(((4 * m + 255) // 256) * 256
                                                             for m in mats)
    # TINY has d_r = 8 and d_cq = 48: no tiled layout
    t = lib.make_config(inputs.TINY, 64, "f32")
    assert lib.packed_weights_size(t) == 0
    p = ctypes.c_void_p(1 << 20)
    src = lib.Weights(*([4096] * 8))
    out = lib.Weights()
    pk = L.mla_pack_weights
    assert pk(ctypes.byref(t), ctypes.byref(src), p, 1 << 40, ctypes.byref(out), None) == lib.MLA_ERR_UNSUPPORTED
    assert pk(None, ctypes.byref(src), p, 1 << 40, ctypes.byref(out), None) == lib.MLA_ERR_INVALID_ARG
    assert pk(ctypes.byref(c), None, p, 1 << 40, ctypes.byref(out), None) == lib.MLA_ERR_INVALID_ARG
    assert pk(ctypes.byref(c), ctypes.byref(src), p, 1 << 40, None, None) == lib.MLA_ERR_INVALID_ARG
    tiled = lib.Weights(*([4096] * 8), lib.LAYOUT_TILES)
    assert pk(ctypes.byref(c), ctypes.byref(tiled), p, 1 << 40, ctypes.byref(out), None) == lib.MLA_ERR_INVALID_ARG
    assert pk(ctypes.byref(c), ctypes.byref(src), p, need - 1, ctypes.byref(out), None) == lib.MLA_ERR_WORKSPACE
    assert pk(ctypes.byref(c), ctypes.byref(src), None, 1 << 40, ctypes.byref(out), None) == lib.MLA_ERR_WORKSPACE
    assert pk(ctypes.byref(c), ctypes.byref(src), ctypes.c_void_p((1 << 20) + 64), 1 << 40,
              ctypes.byref(out), None) == lib.MLA_ERR_WORKSPACE
    # destination overlapping a source matrix
    ov = lib.Weights(*([None] * 7), (1 << 20) + 4096)
    assert pk(ctypes.byref(c), ctypes.byref(ov), p, 1 << 40, ctypes.byref(out), None) == lib.MLA_ERR_INVALID_ARG
    # entry points reject an unknown layout, and tiles on a geometry without them
    z = ctypes.c_void_p(4096)
    bad = lib.Weights(*([4096] * 8), 2)
    assert L.mla_decode_output(ctypes.byref(c), ctypes.byref(bad), z, 1, z, 1 << 40, z, None) == lib.MLA_ERR_INVALID_ARG
    tt = lib.Weights(*([4096] * 8), lib.LAYOUT_TILES)
    assert L.mla_decode_output(ctypes.byref(t), ctypes.byref(tt), z, 1, z, 1 << 40, z, None) == lib.MLA_ERR_UNSUPPORTED
    assert L.mla_append_kv(ctypes.byref(t), ctypes.byref(tt), z, z, z, 3, z, 10, z, 1, z, 1 << 30,
                           None) == lib.MLA_ERR_UNSUPPORTED


def test_merged_entry_points_reject_bad_arguments(L):
    """mla_merge_weights and mla_decode_merged check everything on the host."""
    c = _cfg()
    p = ctypes.c_void_p(1 << 20)
    src = lib.Weights(*([4096] * 8))
    mg = L.mla_merge_weights
    assert mg(ctypes.byref(c), None, 0, p, p, None) == lib.MLA_ERR_INVALID_ARG
    assert mg(ctypes.byref(c), ctypes.byref(src), 0, None, p, None) == lib.MLA_ERR_INVALID_ARG
    assert mg(ctypes.byref(c), ctypes.byref(src), 2, p, p, None) == lib.MLA_ERR_INVALID_ARG
    tiled = lib.Weights(*([4096] * 8), lib.LAYOUT_TILES)
    assert mg(ctypes.byref(c), ctypes.byref(tiled), 0, p, p, None) == lib.MLA_ERR_INVALID_ARG
    no_uv = lib.Weights(4096, 4096, 4096, 4096, 4096, 4096, None, 4096)
    assert mg(ctypes.byref(c), ctypes.byref(no_uv), 0, p, p, None) == lib.MLA_ERR_INVALID_ARG
    t = lib.make_config(inputs.TINY, 64, "f32")
    assert mg(ctypes.byref(t), ctypes.byref(src), lib.LAYOUT_TILES, p, p, None) == lib.MLA_ERR_UNSUPPORTED
    # merged decode: workspace size, weights and arguments
    assert lib.workspace_size(c, lib.OP_DECODE_MERGED, 64, 8193, 0) > 0
    assert lib.workspace_size(t, lib.OP_DECODE_MERGED, 3, 40, 0) > 0
    dm = L.mla_decode_merged
    mw = lib.MergedWeights(4096, 4096, 4096, None, 0)
    z = ctypes.c_void_p(4096)
    assert dm(ctypes.byref(c), ctypes.byref(mw), z, z, z, 4, z, 2, z, 1, 100, z, 10, 0, z, 1 << 40,
              z, None) == lib.MLA_ERR_INVALID_ARG
    mw = lib.MergedWeights(4096, 4096, 4096, 4096, 0)
    # max_kv_len beyond the page table's reach, workspace too small
    assert dm(ctypes.byref(c), ctypes.byref(mw), z, z, z, 4, z, 2, z, 1, 129, z, 200, 0, z, 1 << 40,
              z, None) == lib.MLA_ERR_INVALID_ARG
    assert dm(ctypes.byref(c), ctypes.byref(mw), z, z, z, 4, z, 2, z, 1, 100, z, 200, 0, z, 16,
              z, None) == lib.MLA_ERR_WORKSPACE
    mt = lib.MergedWeights(4096, 4096, 4096, 4096, lib.LAYOUT_TILES)
    assert dm(ctypes.byref(t), ctypes.byref(mt), z, z, z, 4, z, 2, z, 1, 100, z, 200, 0, z, 1 << 40,
              z, None) == lib.MLA_ERR_UNSUPPORTED
    assert dm(ctypes.byref(c), ctypes.byref(mw), None, None, None, 0, None, 0, None, 0, 0, None, 0,
              0, None, 0, None, None) == 0


def test_backward_and_mha_reject_bad_arguments(L):
    c = _cfg()
    p = ctypes.c_void_p(4096)
    wf = lib.Weights(*([4096] * 8))
    bw = L.mla_attention_backward
    args = lambda **kw: [kw.get(k, v) for k, v in (  # noqa: E731
        ("cfg", ctypes.byref(c)), ("w", ctypes.byref(wf)), ("q", p), ("pos", p), ("cache", p),
        ("np", 4), ("pt", p), ("mp", 2), ("kv", 100), ("T", 3), ("dO", p), ("ws", p),
        ("wsb", 1 << 40), ("dWk", p), ("dWv", p), ("dq", p), ("dC", p), ("s", None))]
    assert bw(*args(w=None)) == lib.MLA_ERR_INVALID_ARG
    assert bw(*args(kv=129)) == lib.MLA_ERR_INVALID_ARG           # past the page table
    assert bw(*args(dq=None)) == lib.MLA_ERR_INVALID_ARG
    assert bw(*args(wsb=16)) == lib.MLA_ERR_WORKSPACE
    assert bw(*args(T=0)) == 0
    assert lib.workspace_size(c, lib.OP_ATTENTION_BACKWARD, 64, 64, 0) > 2 * 128 * 64 * 64 * 4
    # MHA baseline: d_h without a power-of-two count of 16-wide pieces
    odd = lib.make_config(inputs.Shape(d=64, n_h=4, d_h=48, d_c=32, d_cq=64, d_r=16), 64, "f32")
    mh = L.mla_mha_decode_attention
    assert mh(ctypes.byref(odd), p, p, 4, p, 2, p, 1, 100, ctypes.c_float(0.0), 0, p, 1 << 40, p,
              None) == lib.MLA_ERR_UNSUPPORTED
    assert mh(ctypes.byref(c), p, ctypes.c_void_p(4096 + 8), 4, p, 2, p, 1, 100,
              ctypes.c_float(0.0), 0, p, 1 << 40, p, None) == lib.MLA_ERR_INVALID_ARG
    assert mh(ctypes.byref(c), p, p, 4, p, 2, p, 1, 100, ctypes.c_float(0.0), 0, p, 16, p,
              None) == lib.MLA_ERR_WORKSPACE


def test_decode_noalloc_host_checks(L):
    """mla_decode_noalloc validates its arguments and its scratch limit on the
    host before any HIP call (this runs without a GPU)."""
    c = _cfg()
    p = ctypes.c_void_p(4096)
    z = ctypes.c_void_p(0)
    wf = lib.Weights(*([4096] * 8))
    wn = lib.Weights(*([None] * 8))
    # null weights, missing output
    assert L.mla_decode_noalloc(ctypes.byref(c), ctypes.byref(wn), p, p, p, 300, p, 129, p, 4,
                                8193, p, 8194, 0, p, None) == lib.MLA_ERR_INVALID_ARG
    assert L.mla_decode_noalloc(ctypes.byref(c), ctypes.byref(wf), p, p, p, 300, p, 129, p, 4,
                                8193, p, 8194, 0, z, None) == lib.MLA_ERR_INVALID_ARG
    # batch 128 with automatic splits needs more than the 64 MiB array
    need = lib.workspace_size(c, lib.OP_DECODE, 128, 8193, 0)
    assert need > 64 << 20
    assert L.mla_decode_noalloc(ctypes.byref(c), ctypes.byref(wf), p, p, p, 300, p, 129, p, 128,
                                8193, p, 8194, 0, p, None) == lib.MLA_ERR_SCRATCH_LIMIT
    # batch 64 fits (the call would launch: not made here); an empty batch is a no-op
    assert lib.workspace_size(c, lib.OP_DECODE, 64, 8193, 0) <= 64 << 20
    assert L.mla_decode_noalloc(ctypes.byref(c), ctypes.byref(wf), p, p, p, 300, p, 129, p, 0,
                                8193, p, 8194, 0, p, None) == lib.MLA_OK
