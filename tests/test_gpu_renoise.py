"""Re-noise on the GPU: bit-exact against the oracle given identical confidences."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_denoise_amd import dgpass
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,N,V", [(1, 256, 32768), (8, 256, 32768), (3, 37, 1000), (64, 5, 1024),
                                   (1, 1, 7), (2, 4099, 1 << 20)])
def test_renoise_bit_exact(B, N, V):
    rng = np.random.default_rng(B * 1000 + N)
    canvas = rng.integers(0, V, (B, N)).astype(np.int32)
    am = rng.integers(0, V, (B, N)).astype(np.int32)
    conf = rng.random((B, N)).astype(np.float32)
    conf.ravel()[::7] = np.nan
    conf.ravel()[::11] = 0.5
    pos0 = rng.integers(0, 100000, B).astype(np.int32)
    req = rng.integers(0, 2**32, B, dtype=np.uint64).astype(np.uint32)
    for seed, tag, tau, use_conf, use_req in [(0, 0, 0.5, False, False), (12345, 3, 0.5, True, True),
                                              (2**63 + 5, 0xFFFFFFFF, 0.0, True, False),
                                              (7, 1, 1.5, True, True)]:
        exp = oracle.renoise(canvas, am if use_conf else None, conf if use_conf else None, tau, seed,
                             tag, pos0, V, req_id=req if use_req else None)
        g = torch.from_numpy(canvas).to(DEV)
        dgpass.renoise(g, torch.from_numpy(am).to(DEV) if use_conf else None,
                       torch.from_numpy(conf).to(DEV) if use_conf else None, tau, seed, tag, pos0, V,
                       req_id=req if use_req else None)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(g.cpu().numpy(), exp)


def test_renoise_in_place_keeps_above_threshold_slots():
    B, N, V = 2, 300, 32768
    rng = np.random.default_rng(9)
    am = torch.from_numpy(rng.integers(0, V, (B, N)).astype(np.int32)).to(DEV)
    conf = torch.from_numpy(rng.random((B, N)).astype(np.float32)).to(DEV)
    canvas = torch.zeros(B, N, dtype=torch.int32, device=DEV)
    dgpass.renoise(canvas, am, conf, 0.7, 1, 2, [0, 256], V)
    keep = conf >= 0.7
    assert torch.equal(canvas[keep], am[keep])
    assert (canvas[~keep] != am[~keep]).float().mean() > 0.99
