"""mla_decode inside a captured HIP graph: the step allocates nothing and
clears no memory with memset nodes, so a captured call replays to the eager
result bit for bit.  The graph is replayed several times with eager work of
the program between the replays, and every replay is compared.
"""
import numpy as np
import pytest
import torch

from mla_latent_kv_15_amd import device, inputs, lib
from tests.gpu_helpers import Layer, cache_from_rows, log, require_lib
from tests.test_gpu_tiles import _bits, _pack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


def test_decode_graph_replays_match_eager():
    s = inputs.V2
    layer = Layer(s, 61, "bf16", keep_host=False)
    B = 16
    L = inputs.make_lengths(B, 200, 2500, 61)
    kv = (L + 1).astype(np.int32)
    paged = inputs.make_paged(kv, 64, 61, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(kv)[:-1]]).astype(np.int64)
    rows = inputs.make_cache_rows(int(kv.sum()), s, 61, "bf16")
    cache = cache_from_rows(layer, rows, paged, offs)
    rope = layer.rope(int(kv.max()) + 1)
    _buf, wt = _pack(layer)
    mx = int(kv.max())
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
    pos, kvd, pt = i32(L), i32(kv), i32(paged.page_table)
    h = device.tensor(inputs.make_hidden(B, s, 61, "bf16"))
    ws = device.workspace(lib.workspace_size(layer.cfg, lib.OP_DECODE, B, mx, 0))
    out = torch.empty(B, s.d, dtype=torch.bfloat16, device="cuda")

    def step(hh, o):
        lib.decode(layer.cfg, wt, hh, pos, cache, pt, kvd, mx, rope, 0, ws, o)

    step(h, out)
    torch.cuda.synchronize()
    ref = _bits(out)
    log("capture mla_decode")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        step(h, out)
    # eager work between the replays: another batch through the same workspace
    h2 = device.tensor(inputs.make_hidden(B, s, 62, "bf16"))
    other = torch.empty_like(out)
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), ref), f"replay {r}"
        step(h2, other)
        torch.cuda.synchronize()
    assert np.isfinite(device.to_f64(out)).all()
