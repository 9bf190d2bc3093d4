"""dg_denoise_pass_next on the GPU: a pass whose last kernel also writes the
expert coverage and re-noises the canvas for the next pass.

Its argmax and conf are those of dg_denoise_pass (the same kernels: bit-exact),
its coverage that of dg_expert_coverage, and its canvas the oracle's re-noise
(explainer "DiffusionGemma", "Uniform State Diffusion"; Philox4x64-10) of the
argmax and conf the pass returned: bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_denoise_amd import dgpass, synth
from block_diffusion_lm_denoise_amd.configs import ModelConfig
from gpu_helpers import DEV, Pair, host

pytestmark = pytest.mark.gpu

CFGS = {
    "bf16": ModelConfig(L=2, D=256, Hq=4, Hkv=2, hd=64, E=16, k=4, F=128, V=1000, act="bf16", expert="bf16"),
    "f32": ModelConfig(L=1, D=128, Hq=2, Hkv=1, hd=64, E=8, k=2, F=128, V=512, act="f32", expert="f32"),
    # rows longer than the 2048 elements the row kernels hold in registers
    "wide": ModelConfig(L=1, D=2560, Hq=4, Hkv=2, hd=128, E=8, k=2, F=128, V=512, act="bf16", expert="bf16"),
}


@pytest.mark.parametrize("name,B,N,lens,use_req", [("bf16", 2, 16, (5, 9), True), ("f32", 3, 7, (0, 4, 1), False),
                                                   ("bf16", 1, 300, (33,), False)])
def test_pass_next_equals_pass_coverage_renoise(name, B, N, lens, use_req):
    cfg = CFGS[name]
    seed, tau, tag = 5, 0.5, 3
    pair = Pair(cfg, seed, scale_lm=12.0)   # confidences straddle tau
    gm = pair.gm
    cap = max(lens) + N
    kv = gm.kv_cache(B, cap, device=DEV)
    ws = gm.workspace(B * max(max(lens), N), cap, device=DEV)
    for b, P in enumerate(lens):   # request b gets a prefix of P tokens
        if P:
            kb = gm.kv_cache(1, cap, device=DEV)
            gm.kv_prefill(kb, synth.tokens(cfg.V, (1, P), seed + b, name="prompt").to(DEV), ws)
            for l in range(cfg.L):
                kv.k[l][b].copy_(kb.k[l][0])
                kv.v[l][b].copy_(kb.v[l][0])
    kv.lens[:] = np.array(lens, np.int32)
    torch.cuda.synchronize()

    canvas0 = synth.tokens(cfg.V, (B, N), seed, name="canvas").to(DEV)
    pos0 = np.array(lens, np.int32)
    req = np.array([7, 2**32 - 1, 12345][:B], np.uint32) if use_req else None

    # separate calls
    cv_a = canvas0.clone()
    am_a = torch.empty(B, N, dtype=torch.int32, device=DEV)
    cf_a = torch.empty(B, N, dtype=torch.float32, device=DEV)
    tt_a = torch.full((cfg.L,), -1, dtype=torch.int32, device=DEV)
    gm.denoise_pass(kv, cv_a, am_a, cf_a, ws)
    gm.expert_coverage(ws, tt_a)
    dgpass.renoise(cv_a, am_a, cf_a, tau, seed, tag, pos0, cfg.V, req_id=req)
    torch.cuda.synchronize()

    # one call
    cv_b = canvas0.clone()
    am_b = torch.full((B, N), -1, dtype=torch.int32, device=DEV)
    cf_b = torch.full((B, N), -1.0, dtype=torch.float32, device=DEV)
    tt_b = torch.full((cfg.L,), -1, dtype=torch.int32, device=DEV)
    rn = dict(tau=tau, seed=seed, pass_tag=tag, pos0=pos0)
    if req is not None:
        rn["req_id"] = req
    gm.denoise_pass_next(kv, cv_b, am_b, cf_b, ws, touched=tt_b, renoise=rn)
    torch.cuda.synchronize()

    np.testing.assert_array_equal(host(am_b), host(am_a))
    np.testing.assert_array_equal(host(cf_b).view(np.uint32), host(cf_a).view(np.uint32))
    np.testing.assert_array_equal(host(tt_b), host(tt_a))
    np.testing.assert_array_equal(host(cv_b), host(cv_a))
    # the re-noise is the oracle's, applied to the pass's own outputs
    exp = oracle.renoise(host(canvas0), host(am_b), host(cf_b), tau, seed, tag, pos0, cfg.V, req_id=req)
    np.testing.assert_array_equal(host(cv_b), exp)
    kept = host(cf_b) >= tau
    assert 0 < kept.mean() < 1, kept.mean()
    assert 0 < int(host(tt_b).min()) and int(host(tt_b).max()) <= cfg.E


def test_pass_next_without_renoise_leaves_the_canvas():
    cfg = CFGS["f32"]
    pair = Pair(cfg, 11)
    gm = pair.gm
    B, N = 2, 9
    kv = gm.kv_cache(B, N, device=DEV)
    ws = gm.workspace(B * N, N, device=DEV)
    canvas = synth.tokens(cfg.V, (B, N), 11, name="canvas").to(DEV)
    before = host(canvas).copy()
    am = torch.empty(B, N, dtype=torch.int32, device=DEV)
    cf = torch.empty(B, N, dtype=torch.float32, device=DEV)
    am2, cf2 = torch.empty_like(am), torch.empty_like(cf)
    tt = torch.full((cfg.L,), -1, dtype=torch.int32, device=DEV)
    tt2 = torch.full((cfg.L,), -1, dtype=torch.int32, device=DEV)
    gm.denoise_pass_next(kv, canvas, am, cf, ws, touched=tt)          # coverage only
    gm.denoise_pass_next(kv, canvas, am2, cf2, ws)                     # neither: a plain pass
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(canvas), before)
    np.testing.assert_array_equal(host(am), host(am2))
    np.testing.assert_array_equal(host(cf).view(np.uint32), host(cf2).view(np.uint32))
    gm.expert_coverage(ws, tt2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(tt), host(tt2))


@pytest.mark.parametrize("name,sampler,B,N,lens", [("bf16", "uniform", 2, 16, (5, 9)),
                                                   ("bf16", "masked", 1, 300, (33,)),
                                                   ("f32", "uniform", 3, 7, (0, 4, 1)),
                                                   ("wide", "uniform", 1, 24, (11,))])
def test_embedding_carry_equals_embedding_each_pass(name, sampler, B, N, lens):
    """A chain of passes whose last kernel also embeds the updated canvas for
    the next pass (embed_next), the next pass skipping its own embedding
    (input_embedded), gives bit for bit the canvases, argmax, conf, coverage and
    change counts of the same chain embedding the canvas in every pass."""
    cfg = CFGS[name]
    # masked rows see nearly the same context under random weights, so they
    # share one confidence: tau 0 fills them all on the first pass
    seed, tau, S = 9, (0.0 if sampler == "masked" else 0.5), 4
    pair = Pair(cfg, seed, scale_lm=12.0)   # uniform: confidences straddle tau
    gm = pair.gm
    cap = max(lens) + N
    _, _, _, kv = pair.caches(B, cap, list(lens), seed, synthetic=True)
    ws = gm.workspace(B * max(max(lens), N), cap, device=DEV)
    pos0 = np.array(lens, np.int32)
    mask_id = cfg.V - 1
    canvas0 = synth.tokens(cfg.V - 1, (B, N), seed, name="canvas")
    if sampler == "masked":   # every other slot masked: rows differ, so confidences do
        canvas0[:, ::2] = mask_id
    canvas0 = canvas0.to(DEV)

    def chain(carry):
        cv = canvas0.clone()
        ch = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        ml = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        outs, have = [], False
        for p in range(S):
            am = torch.full((B, N), -1, dtype=torch.int32, device=DEV)
            cf = torch.full((B, N), -1.0, dtype=torch.float32, device=DEV)
            tt = torch.full((cfg.L,), -1, dtype=torch.int32, device=DEV)
            ahead = carry and p + 1 < S
            rn = dict(tau=tau, seed=seed, pass_tag=p + 1, pos0=pos0, sampler=sampler, mask_id=mask_id,
                      final_pass=p == S - 1, changed=ch, masked_left=ml, embed_next=ahead,
                      input_embedded=have)
            gm.denoise_pass_next(kv, cv, am, cf, ws, touched=tt, renoise=rn)
            have = ahead
            torch.cuda.synchronize()
            outs.append((host(cv).copy(), host(am).copy(), host(cf).view(np.uint32).copy(),
                         host(tt).copy(), host(ch).copy(), host(ml).copy()))
        return outs

    plain, carried = chain(False), chain(True)
    for p, (a, b) in enumerate(zip(plain, carried)):
        for what, x, y in zip(("canvas", "argmax", "conf", "touched", "changed", "masked_left"), a, b):
            np.testing.assert_array_equal(y, x, err_msg=f"pass {p}: {what}")
    # the chain did change the canvas between passes (the carry had work to do)
    assert any(int(o[4].sum()) > 0 for o in plain[:-1])
