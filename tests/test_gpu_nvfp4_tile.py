"""moe_nvfp4_tile: NVFP4 weights from row-major to the k-tiled layout the
expert GEMMs read (a byte permutation, so checked bit-exactly against the
same permutation written with numpy).  The layout: for each matrix, 64-deep
k-slab t holds every row's 32 code bytes (elements 64t .. 64t + 63, dwords
in the order 0, 2, 4, 6, 1, 3, 5, 7) and 4 block-scale bytes (blocks 4t ..
4t + 3) in row order; the NVFP4 format itself
(E2M1 codes, one E4M3 scale per 16 elements) is that of the Korean Nemotron 3
summary, section 2.4 NVFP4 Training.
"""
import numpy as np
import pytest
import torch

from sparse_moe_layer_fwd_amd import binding as B

pytestmark = pytest.mark.gpu


def _tiled(codes, scales, k):
    # within a row's 32 bytes of a slab, the 8 dwords (8 codes each) go in the
    # order 0, 2, 4, 6, 1, 3, 5, 7
    n, rows = codes.shape[:2]
    ct = codes.reshape(n, rows, k // 64, 8, 4)[:, :, :, [0, 2, 4, 6, 1, 3, 5, 7], :]
    ct = ct.reshape(n, rows, k // 64, 32).transpose(0, 2, 1, 3).reshape(n, -1)
    st = scales.reshape(n, rows, k // 64, 4).transpose(0, 2, 1, 3).reshape(n, -1)
    return ct, st


@pytest.mark.parametrize("n,rows,k", [(1, 1, 64), (3, 40, 192), (5, 257, 1024), (2, 1000, 2688)])
def test_tile_matches_numpy_permutation(n, rows, k):
    rng = np.random.default_rng(rows + k)
    codes = rng.integers(0, 256, size=(n, rows, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(n, rows, k // 16), dtype=np.uint8)
    dev = torch.device("cuda")
    c_in, s_in = torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev)
    c_out = torch.full_like(c_in, 0x5A)
    s_out = torch.full_like(s_in, 0x5A)
    B.moe_nvfp4_tile(c_in.data_ptr(), s_in.data_ptr(), c_out.data_ptr(), s_out.data_ptr(), n, rows, k,
                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ct, st = _tiled(codes, scales, k)
    assert np.array_equal(c_out.cpu().numpy().reshape(n, -1), ct)
    assert np.array_equal(s_out.cpu().numpy().reshape(n, -1), st)
    # the inputs are left alone
    assert np.array_equal(c_in.cpu().numpy(), codes) and np.array_equal(s_in.cpu().numpy(), scales)
