"""mla_decode_noalloc (the decode step on the library's fixed device scratch
array) against mla_decode on a caller workspace: bit-identical outputs, for
two calls in a row, the second with a smaller batch."""
import numpy as np
import pytest
import torch

from mla_latent_kv_15_amd import device, inputs, lib
from tests.gpu_helpers import Layer, cache_from_rows, log, require_lib

pytestmark = pytest.mark.gpu


def _case(layer, wts, B, cid):
    s = inputs.V2
    L = inputs.make_lengths(B, 100, 3000, cid)
    kv = (L + 1).astype(np.int32)
    paged = inputs.make_paged(kv, 64, cid, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(kv)[:-1]]).astype(np.int64)
    rows = inputs.make_cache_rows(int(kv.sum()), s, cid, "bf16")
    cache = cache_from_rows(layer, rows, paged, offs)
    h = device.tensor(inputs.make_hidden(B, s, cid, "bf16"))
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
    return dict(h=h, pos=i32(L), kv=i32(kv), pt=i32(paged.page_table), cache=cache,
                max_kv=int(kv.max()))


def test_decode_noalloc_matches_decode():
    require_lib()
    s = inputs.V2
    layer = Layer(s, 41, "bf16", keep_host=False)
    packed = device.workspace(lib.packed_weights_size(layer.cfg))
    wts = lib.pack_weights(layer.cfg, layer.wts, packed)
    rope = layer.rope(3100)
    for B, cid in ((12, 41), (3, 42)):   # the second call is smaller than the first
        log(f"no-alloc decode: batch {B}")
        c = _case(layer, wts, B, cid)
        ws = device.workspace(lib.workspace_size(layer.cfg, lib.OP_DECODE, B, c["max_kv"], 0))
        ref = torch.empty(B, s.d, dtype=torch.bfloat16, device="cuda")
        out = torch.full((B, s.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lib.decode(layer.cfg, wts, c["h"], c["pos"], c["cache"], c["pt"], c["kv"], c["max_kv"],
                   rope, 0, ws, ref)
        lib.decode_noalloc(layer.cfg, wts, c["h"], c["pos"], c["cache"], c["pt"], c["kv"],
                           c["max_kv"], rope, 0, out)
        torch.cuda.synchronize()
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), B
