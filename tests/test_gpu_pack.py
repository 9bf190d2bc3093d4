"""The packed weight layout written on the GPU, bit for bit against the
layout's definition (tiles of 16 rows x 128 bytes; half h, lane l of a tile
holds row 16 rg + l % 16, bytes 128 kb + 64 h + 16 (l / 16) .. +15)."""
import numpy as np
import pytest
import torch

from block_diffusion_lm_denoise_amd import dgpass

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed_reference(src: np.ndarray) -> np.ndarray:
    """src: uint8 [rows][rowbytes] -> packed bytes, from the definition."""
    rows, rb = src.shape
    nkb, nrg = rb // 128, (rows + 15) // 16
    pad = np.zeros((nrg * 16, rb), np.uint8)
    pad[:rows] = src
    out = np.zeros(nrg * nkb * 2048, np.uint8)
    for rg in range(nrg):
        for kb in range(nkb):
            base = (rg * nkb + kb) * 2048
            for h in range(2):
                for l in range(64):
                    r, c = 16 * rg + l % 16, 128 * kb + 64 * h + 16 * (l // 16)
                    o = base + 1024 * h + 16 * l
                    out[o:o + 16] = pad[r, c:c + 16]
    return out


@pytest.mark.parametrize("rows,cols,dtype,es", [(16, 64, "bf16", 2), (40, 256, "bf16", 2),
                                                (33, 128, "fp8", 1), (8, 96, "f32", 4),
                                                (48, 384, "fp8", 1)])
def test_pack_matches_the_layout_definition(rows, cols, dtype, es):
    rng = np.random.default_rng(rows * 1000 + cols)
    src = rng.integers(0, 256, size=(rows, cols * es), dtype=np.uint8)
    d = torch.from_numpy(src).to(DEV)
    p = dgpass.pack_weight(d, rows, cols, dtype)
    torch.cuda.synchronize()
    got = p.cpu().numpy()
    assert got.size == dgpass.packed_bytes(rows, cols, dtype)
    np.testing.assert_array_equal(got, packed_reference(src))


def test_pack_of_a_large_matrix_sampled():
    # LM-head sized: 32768 x 2048 bf16; check whole tiles at sampled positions
    rows, cols = 32768, 2048
    g = torch.Generator(device=DEV).manual_seed(7)
    src = torch.randint(0, 256, (rows, cols * 2), dtype=torch.uint8, device=DEV, generator=g)
    p = dgpass.pack_weight(src, rows, cols, "bf16").cpu().numpy()
    s = src.cpu().numpy()
    nkb = cols * 2 // 128
    for rg, kb in [(0, 0), (0, nkb - 1), (1234, 17), (rows // 16 - 1, nkb - 1)]:
        tile = p[(rg * nkb + kb) * 2048:(rg * nkb + kb + 1) * 2048]
        ref = packed_reference(s[16 * rg:16 * rg + 16, 128 * kb:128 * kb + 128])
        np.testing.assert_array_equal(tile, ref)
