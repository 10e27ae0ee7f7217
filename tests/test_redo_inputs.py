"""CPU check of the softmax redo test's inputs: without the redo (or with a
redo that only some heads can request) the planted scores overflow fp32."""
import numpy as np

from mla_latent_kv_15_amd import inputs
from tests.jump_rows import JUMP_LENS, JUMPS, plant_jumps, rand_q


def test_jump_rows_overflow_without_redo():
    s = inputs.V2
    lens = JUMP_LENS
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = inputs.make_cache_rows(int(lens.sum()), s, 27, "bf16")
    qa = rand_q(len(lens), s, 27)
    f32 = rows.f32.copy()
    plant_jumps(qa.f32, f32, offs)
    r64 = inputs.Array(f32, "bf16").f64()
    q64 = qa.f64()
    for b, hd, t in JUMPS:
        sc = q64[b][hd] @ r64[offs[b]:offs[b] + lens[b]].T
        rest = np.delete(sc, t)
        # e^(s_t - max of the rest) > 2^144: beyond fp32 (2^128) whatever
        # the segment's first 32 scores were
        assert (sc[t] - rest.max()) / np.log(2.0) > 144, (b, hd)
        assert t % 64 >= 32 and t < lens[b]
