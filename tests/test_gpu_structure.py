"""GPU structural checks: paging and indexing bit-exact, kv_len edges, split
invariance, append slot discipline, invalid device indices."""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_15_amd import device, inputs
from tests.gpu_helpers import TOL, Layer, cache_from_rows, log, require_lib
from tests.jump_rows import JUMP_LENS, plant_jumps, rand_q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


@pytest.fixture(scope="module")
def v2():
    return Layer(inputs.V2, 21, "bf16")


EDGE_LENS = [1, 2, 63, 64, 65, 127, 128, 129, 1000, 4097]


def test_kv_len_edges_against_oracle(v2):
    s = inputs.V2
    lens = np.array(EDGE_LENS, np.int32)
    B = len(lens)
    paged = inputs.make_paged(lens, 64, 22, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 22, "bf16")
    cache = cache_from_rows(v2, rows, paged, offs)
    qa = rand_q(B, s, 22)
    for ns in (0, 1, 2, 7):
        log(f"edges: splits {ns}")
        lat = device.to_f64(v2.decode_attention(device.tensor(qa), cache, paged.page_table, lens,
                                                int(lens.max()), ns))
        r64 = rows.f64()
        for b in range(B):
            ref = oracle.latent_attention(qa.f64()[b], r64[offs[b]:offs[b] + lens[b]], s.d_c)
            err = oracle.max_rel_error(lat[b], ref)
            assert err < TOL["bf16"], (lens[b], ns, err)


def test_page_permutation_bit_exact(v2):
    """Same rows, different physical pages: bit-identical outputs."""
    s = inputs.V2
    lens = np.array([1, 64, 65, 700, 3000], np.int32)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 23, "bf16")
    qa = device.tensor(rand_q(len(lens), s, 23))
    outs = []
    for shuffle, extra in ((False, 0), (True, 0), (True, 9)):
        paged = inputs.make_paged(lens, 64, 23 + extra, shuffle=shuffle, extra_pages=extra)
        cache = cache_from_rows(v2, rows, paged, offs)
        outs.append(v2.decode_attention(qa, cache, paged.page_table, lens, int(lens.max()), 0))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_split_invariance(v2):
    s = inputs.V2
    lens = np.array([5000, 130, 4097, 64], np.int32)
    paged = inputs.make_paged(lens, 64, 24, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 24, "bf16")
    cache = cache_from_rows(v2, rows, paged, offs)
    qa = device.tensor(rand_q(len(lens), s, 24))
    base = device.to_f64(v2.decode_attention(qa, cache, paged.page_table, lens, 5000, 1))
    for ns in (2, 7, 64, 0):
        o = device.to_f64(v2.decode_attention(qa, cache, paged.page_table, lens, 5000, ns))
        assert oracle.max_rel_error(o, base) < 1e-2


def test_append_writes_only_its_slots():
    s = inputs.TINY
    layer = Layer(s, 25, "f32", page=4)
    T = 6
    H = inputs.make_hidden(T, s, 25, "f32")
    num_pages = 5
    cache = layer.empty_cache(num_pages, fill=-7.0)
    slots = np.array([3, 4, 17, -1, 19, 10_000], np.int32)   # -1 and 10000 are not written
    rope = layer.rope(32)
    layer.append(device.tensor(H), np.arange(T), slots, cache, rope)
    flat = device.to_f64(cache).reshape(-1, s.row)
    written = {3, 4, 17, 19}
    for slot in range(num_pages * 4):
        if slot not in written:
            assert np.all(flat[slot] == -7.0), slot
    c, kr = oracle.latent_rows(H.f64(), layer.W64["W_DKV"], layer.W64["W_KR"], np.arange(T), 10000.0)
    ref = np.concatenate([c, kr], 1)
    for t, slot in enumerate(slots):
        if slot in written:
            assert oracle.max_rel_error(flat[slot], ref[t]) < 1e-5


def test_invalid_device_indices_give_nan_rows(v2):
    s = inputs.V2
    lens = np.array([100, 100, 100, 100], np.int32)
    paged = inputs.make_paged(lens, 64, 26, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 26, "bf16")
    cache = cache_from_rows(v2, rows, paged, offs)
    qa = rand_q(4, s, 26)
    pt = paged.page_table.copy()
    pt[1, 1] = paged.num_pages + 5        # page id out of range
    bad_lens = lens.copy()
    bad_lens[2] = 0                       # kv_len below 1
    bad_lens[3] = 129                     # beyond the page table row (2 pages)
    lat = device.to_f64(v2.decode_attention(device.tensor(qa), cache, pt, bad_lens, 128, 0))
    assert np.all(np.isnan(lat[1])) and np.all(np.isnan(lat[2])) and np.all(np.isnan(lat[3]))
    ref = oracle.latent_attention(qa.f64()[0], rows.f64()[:100], s.d_c)
    assert oracle.max_rel_error(lat[0], ref) < TOL["bf16"]


def test_score_jump_redo_path(v2):
    """Scores far above a segment's first scores, on heads that are and are
    not the first head of a wave: the exact-max redo keeps every output
    finite and equal to the oracle's, for automatic and forced splits."""
    s = inputs.V2
    lens = JUMP_LENS
    paged = inputs.make_paged(lens, 64, 27, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 27, "bf16")
    qa = rand_q(len(lens), s, 27)
    f32 = rows.f32.copy()
    plant_jumps(qa.f32, f32, offs)
    rows = inputs.Array(f32, "bf16")
    cache = cache_from_rows(v2, rows, paged, offs)
    r64 = rows.f64()
    refs = [oracle.latent_attention(qa.f64()[b], r64[offs[b]:offs[b] + lens[b]], s.d_c)
            for b in range(len(lens))]
    for ns in (0, 1, 7):
        log(f"redo: splits {ns}")
        lat = device.to_f64(v2.decode_attention(device.tensor(qa), cache, paged.page_table, lens,
                                                int(lens.max()), ns))
        assert np.all(np.isfinite(lat)), ns
        for b in range(len(lens)):
            err = oracle.max_rel_error(lat[b], refs[b])
            assert err < TOL["bf16"], (ns, b, err)


def test_many_sequences_mixed_lengths(v2):
    """More sequences than the planner handles in one pass, with invalid
    lengths mixed in: sampled rows match the oracle, invalid rows are NaN,
    and the auto split agrees with one segment per sequence."""
    s = inputs.V2
    rng = np.random.default_rng(28)
    B = 300
    lens = rng.integers(1, 400, B).astype(np.int32)
    lens[rng.choice(B, 40, replace=False)] = rng.integers(1, 8, 40)   # short ones
    paged = inputs.make_paged(lens, 64, 28, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 28, "bf16")
    cache = cache_from_rows(v2, rows, paged, offs)
    qa = rand_q(B, s, 28)
    bad = lens.copy()
    invalid = [7, 150, 257, 299]
    bad[invalid] = 0
    qd = device.tensor(qa)
    lat0 = device.to_f64(v2.decode_attention(qd, cache, paged.page_table, bad, 400, 0))
    lat1 = device.to_f64(v2.decode_attention(qd, cache, paged.page_table, bad, 400, 1))
    for b in invalid:
        assert np.all(np.isnan(lat0[b])) and np.all(np.isnan(lat1[b])), b
    ok = np.setdiff1d(np.arange(B), invalid)
    # both results round bf16 partials and outputs: they agree to the bf16 bar
    assert oracle.max_rel_error(lat0[ok], lat1[ok]) < TOL["bf16"]
    r64 = rows.f64()
    for b in rng.choice(ok, 12, replace=False).tolist() + [0, 255, 256, 298]:
        ref = oracle.latent_attention(qa.f64()[b], r64[offs[b]:offs[b] + lens[b]], s.d_c)
        for lat in (lat0, lat1):
            err = oracle.max_rel_error(lat[b], ref)
            assert err < TOL["bf16"], (b, lens[b], err)


@pytest.mark.parametrize("page", [128, 192])
def test_v2_pages_larger_than_64(page):
    """The MFMA attention accepts any page that is a multiple of 64 tokens:
    page windows, the next segment's first sub-tiles and the in-page offset
    wrap are checked against the oracle at 128- and 192-token pages."""
    s = inputs.V2
    layer = Layer(s, 29, "bf16", page=page)
    lens = np.array([1, 63, 64, 65, page - 1, page, page + 1, 3 * page + 40, 5000, 9000], np.int32)
    paged = inputs.make_paged(lens, page, 29 + page, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 29, "bf16")
    cache = cache_from_rows(layer, rows, paged, offs)
    qa = rand_q(len(lens), s, 29)
    r64 = rows.f64()
    refs = [oracle.latent_attention(qa.f64()[b], r64[offs[b]:offs[b] + lens[b]], s.d_c)
            for b in range(len(lens))]
    for ns in (0, 1, 3, 40):
        log(f"page {page}: splits {ns}")
        lat = device.to_f64(layer.decode_attention(device.tensor(qa), cache, paged.page_table,
                                                   lens, int(lens.max()), ns))
        for b in range(len(lens)):
            err = oracle.max_rel_error(lat[b], refs[b])
            assert err < TOL["bf16"], (page, ns, int(lens[b]), err)


def test_merge_more_than_64_segments_per_sequence(v2):
    """Batches of 32 and more merge in combine_v2_kernel, whose segment
    weights are staged 64 segments at a time: sequences cut into 66 to 120
    segments (120 forced splits) and one 131073-token sequence beside 31 short ones
    (automatic plan) take the multi-pass branch; sampled sequences match the
    oracle and the forced split agrees with one segment per sequence."""
    s = inputs.V2
    rng = np.random.default_rng(30)
    B = 32
    # forced: 120 splits of at most 120 tiles of 64 tokens -> one segment per
    # tile (66..120 per sequence)
    lens = rng.integers(66 * 64 - 63, 120 * 64 + 1, B).astype(np.int32)
    paged = inputs.make_paged(lens, 64, 30, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 30, "bf16")
    cache = cache_from_rows(v2, rows, paged, offs)
    qa = rand_q(B, s, 30)
    qd = device.tensor(qa)
    log("merge: forced 120 splits")
    lat = device.to_f64(v2.decode_attention(qd, cache, paged.page_table, lens, int(lens.max()), 120))
    one = device.to_f64(v2.decode_attention(qd, cache, paged.page_table, lens, int(lens.max()), 1))
    assert oracle.max_rel_error(lat, one) < TOL["bf16"]
    r64 = rows.f64()
    for b in [0, 7, 31] + rng.choice(B, 3, replace=False).tolist():
        ref = oracle.latent_attention(qa.f64()[b], r64[offs[b]:offs[b] + lens[b]], s.d_c)
        err = oracle.max_rel_error(lat[b], ref)
        assert err < TOL["bf16"], (b, int(lens[b]), err)
    del cache, rows, r64
    # automatic plan: the long sequence spreads over most work-groups
    lens = rng.integers(1, 300, B).astype(np.int32)
    lens[13] = 131073
    paged = inputs.make_paged(lens, 64, 31, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 31, "bf16")
    cache = cache_from_rows(v2, rows, paged, offs)
    qa = rand_q(B, s, 31)
    log("merge: automatic plan, one 131073-token sequence")
    lat = device.to_f64(v2.decode_attention(device.tensor(qa), cache, paged.page_table, lens,
                                            int(lens.max()), 0))
    r64 = rows.f64()
    for b in (13, 0, 31, 5):
        ref = oracle.latent_attention(qa.f64()[b], r64[offs[b]:offs[b] + lens[b]], s.d_c)
        err = oracle.max_rel_error(lat[b], ref)
        assert err < TOL["bf16"], (b, int(lens[b]), err)
