"""moe_forward_noalloc (the library's own scratch array as the workspace)
against moe_forward (a caller workspace): the same kernels, so bitwise the
same y, indices, gates and counts, on two calls in a row on one GPU, the second
with fewer tokens than the first; and the size limit of the scratch array.
"""
import pytest
import torch

from test_gpu_parity import SMALL, log, prepare
from sparse_moe_layer_fwd_amd import binding as B

pytestmark = pytest.mark.gpu


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.parametrize("name,t2", [("decode_bf16", 20), ("decode_nvfp4", 33), ("std_shared", 77),
                                     ("hot_cold_nvfp4", 300), ("router_on_x_shared", 129)])
def test_noalloc_matches_forward_twice(name, t2):
    cfg = SMALL[name]
    log("case noalloc %s T=%d then %d" % (name, cfg.T, t2))
    wl, dl, x = prepare(cfg, 2, margin=False)
    assert dl.workspace_bytes(cfg.T) <= B.MOE_SCRATCH_BYTES
    for T in (cfg.T, t2):
        xs = x[:T].contiguous()
        got = dl.forward_noalloc(xs, routing=True)
        torch.cuda.synchronize()
        ref = dl.forward(xs, routing=True)
        torch.cuda.synchronize()
        for g, r, what in zip(got, ref, ("y", "idx", "gate", "counts")):
            assert _same(g, r), "%s differs at T=%d" % (what, T)


def test_noalloc_rejects_a_batch_beyond_the_scratch_array():
    cfg = SMALL["multi_item_256"]
    wl, dl, x = prepare(cfg, 0, margin=False)
    big = cfg.T
    assert dl.workspace_bytes(big) > B.MOE_SCRATCH_BYTES
    y = torch.empty((big, cfg.d), dtype=torch.bfloat16, device=x.device)
    s = torch.cuda.current_stream().cuda_stream
    st = B.moe_forward_noalloc(dl.handle, x.data_ptr(), big, y.data_ptr(), None, None, None, s,
                               check=False)
    assert st == B.MOE_ERR_WORKSPACE
    # a batch that fits still runs, bitwise as moe_forward
    small = 2048
    assert dl.workspace_bytes(small) <= B.MOE_SCRATCH_BYTES
    xs = x[:small].contiguous()
    y1 = dl.forward_noalloc(xs)
    y2 = dl.forward(xs)
    torch.cuda.synchronize()
    assert _same(y1, y2)
