"""Cached rows planted so that one head's score jumps far above the rest of
its segment (inputs of the softmax redo test; no GPU needed here)."""
import numpy as np

from mla_latent_kv_15_amd import inputs

JUMP_LENS = np.array([300, 5000, 2200, 1100], np.int32)
# (sequence, head, token).  Heads 5, 77 and 127 are not the first head of a
# 32-head group, head 0 and 64 are.  Every token has t % 64 >= 32: segments
# start on 64-token boundaries, so the row never falls among the first 32
# scores of a segment.
JUMPS = [(0, 5, 250), (1, 77, 4321), (1, 127, 2150), (2, 0, 1000), (3, 64, 700)]
JUMP_NATS = 110.0


def rand_q(B, s, cid, std=1.0):
    """A random absorbed query with elements of the absorbed query's scale."""
    return inputs.Array(inputs.normal((B, s.n_h, s.row), std * 0.05, cid, inputs.STREAM_QUERY),
                        "bf16")


def plant_jumps(q, f32, offs):
    """Row offs[b] + t := sign(q[b][hd]) * J / |q[b][hd]|_1, so head hd's
    score of that row is J nats (before bf16 rounding of the row)."""
    for b, hd, t in JUMPS:
        f32[offs[b] + t] = np.sign(q[b][hd]) * JUMP_NATS / np.abs(q[b][hd]).sum()
