"""Block chaining on the GPU (driver.generate: prompt prefill, canvases of S
passes with re-noise between passes, commit, append prefill) against the same
loop written over the oracle.

Explainer "DiffusionGemma", sections "Uniform State Diffusion" and "Long-form
text: chaining canvases".  With fp32 storage the two sides agree to ~1e-6, so
every argmax and routing decision is the same unless two logits tie to that
precision; the free-running chains are then identical: committed canvases and
expert coverage bit-exact, caches within the fp32 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_denoise_amd import driver, synth
from block_diffusion_lm_denoise_amd.configs import ModelConfig
from gpu_helpers import DEV, TOL, Pair, f64, host, max_rel

pytestmark = pytest.mark.gpu


def oracle_generate(om, cfg, prompt, n_canvases, N, S, tau, seed):
    B, P = prompt.shape
    ks, vs = om.new_cache(B, P + n_canvases * N)
    lens = np.zeros(B, np.int32)
    if P:
        om.kv_prefill(ks, vs, lens, prompt)
    commits, touched, kept = [], [], []
    for _ in range(n_canvases):
        pos0 = lens.copy()
        canvas = oracle.renoise(np.zeros((B, N), np.int32), None, None, tau, seed, 0, pos0, cfg.V)
        per_pass = []
        for p in range(S):
            am, cf, t = om.denoise_pass(ks, vs, lens, canvas, taps=("counts",))
            per_pass.append((t["counts"] > 0).sum(axis=1))
            kept.append(float((cf >= tau).mean()))
            if p < S - 1:
                canvas = oracle.renoise(canvas, am, cf, tau, seed, p + 1, pos0, cfg.V)
        commits.append(am.copy())
        om.kv_prefill(ks, vs, lens, am)
        touched.append(per_pass)
    return commits, np.array(touched, np.int32), lens, ks, vs, kept


@pytest.mark.parametrize("B,P,N,S,n_canvases", [(2, 7, 16, 3, 2), (1, 0, 9, 2, 3)])
def test_generate_chains_like_the_oracle(B, P, N, S, n_canvases):
    cfg = ModelConfig(L=2, D=256, Hq=4, Hkv=2, hd=64, E=8, k=2, F=128, V=512, act="f32", expert="f32")
    seed, tau = 21, 0.5
    # the head is scaled so that confidences straddle tau: some slots are kept,
    # some re-noised, in every pass
    pair = Pair(cfg, seed, scale_lm=12.0)
    prompt = synth.tokens(cfg.V, (B, P), seed, name="prompt")
    commits, touched, lens, ks, vs, kept = oracle_generate(pair.om, cfg, prompt.numpy(), n_canvases, N, S, tau, seed)

    cap = P + n_canvases * N
    kv = pair.gm.kv_cache(B, cap, device=DEV)
    ws = pair.gm.workspace(max(B * max(P, 1), B * N), cap, device=DEV)
    res = driver.generate(pair.gm, kv, prompt.to(DEV) if P else None, n_canvases, N, S, tau, seed, ws,
                          prefill_prompt=P > 0)
    torch.cuda.synchronize()

    assert len(res.canvases) == n_canvases
    for c in range(n_canvases):
        np.testing.assert_array_equal(host(res.canvases[c]), commits[c], err_msg=f"canvas {c}")
    np.testing.assert_array_equal(host(res.touched), touched)
    assert res.lens == [int(x) for x in lens]
    for l in range(cfg.L):
        for b in range(B):
            n = int(lens[b])
            assert max_rel(f64(host(kv.k[l][b, :, :n]), cfg.act), f64(ks[l][b, :, :n], cfg.act)) < TOL[cfg.act]
            assert max_rel(f64(host(kv.v[l][b, :, :n]), cfg.act), f64(vs[l][b, :, :n], cfg.act)) < TOL[cfg.act]
    # the planted head makes some slots confident and leaves others below tau
    assert 0.0 < float(np.mean(kept)) < 1.0, kept
