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


def oracle_generate(om, cfg, prompt, n_canvases, N, S, tau, seed, sampler="uniform", mask_id=None,
                    early_exit=False):
    """The generation loop over the oracle: the same steps in the same order
    (initial noise or [MASK] canvas; passes with the update between them;
    under early exit, stop once an update changed nothing (uniform) or left
    nothing masked (masked); commit; append prefill)."""
    B, P = prompt.shape
    ks, vs = om.new_cache(B, P + n_canvases * N)
    lens = np.zeros(B, np.int32)
    if P:
        om.kv_prefill(ks, vs, lens, prompt)
    commits, touched, kept, used = [], [], [], []
    for _ in range(n_canvases):
        pos0 = lens.copy()
        if sampler == "uniform":
            canvas = oracle.renoise(np.zeros((B, N), np.int32), None, None, tau, seed, 0, pos0, cfg.V)
        else:
            canvas = np.full((B, N), mask_id, np.int32)
        per_pass = []
        ran = S
        for p in range(S):
            am, cf, t = om.denoise_pass(ks, vs, lens, canvas, taps=("counts",))
            per_pass.append((t["counts"] > 0).sum(axis=1))
            kept.append(float((cf >= tau).mean()))
            last = p == S - 1
            if sampler == "uniform":
                if last:
                    break
                new = oracle.renoise(canvas, am, cf, tau, seed, p + 1, pos0, cfg.V)
                done = (new == canvas).all()
            else:
                new, _, left = oracle.unmask(canvas, am, cf, tau, mask_id, final_pass=last)
                done = (left == 0).all()
            canvas = new
            if early_exit and not last and done:
                ran = p + 1
                break
        commit = am.copy() if sampler == "uniform" else canvas.copy()
        commits.append(commit)
        om.kv_prefill(ks, vs, lens, commit)
        per_pass += [np.zeros(cfg.L, np.int64)] * (S - len(per_pass))
        touched.append(per_pass)
        used.append(ran)
    return commits, np.array(touched, np.int32), lens, ks, vs, kept, used


@pytest.mark.parametrize("B,P,N,S,n_canvases", [(2, 7, 16, 3, 2), (1, 0, 9, 2, 3)])
def test_generate_chains_like_the_oracle(B, P, N, S, n_canvases):
    cfg = ModelConfig(L=2, D=256, Hq=4, Hkv=2, hd=64, E=8, k=2, F=128, V=512, act="f32", expert="f32")
    seed, tau = 21, 0.5
    # the head is scaled so that confidences straddle tau: some slots are kept,
    # some re-noised, in every pass
    pair = Pair(cfg, seed, scale_lm=12.0)
    prompt = synth.tokens(cfg.V, (B, P), seed, name="prompt")
    commits, touched, lens, ks, vs, kept, _ = oracle_generate(pair.om, cfg, prompt.numpy(), n_canvases, N,
                                                              S, tau, seed)

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



@pytest.mark.parametrize("sampler,tau,early_exit", [("masked", 0.5, False), ("masked", 0.3, True),
                                                    ("uniform", 0.0, True), ("uniform", 0.5, True)])
def test_sampler_variants_chain_like_the_oracle(sampler, tau, early_exit):
    """Masked ("absorbing") diffusion and early exit at convergence
    (explainer "DiffusionGemma", "First attempt: masked diffusion" and
    "Uniform State Diffusion"): commits, passes run and coverage equal the
    oracle loop's; under masked diffusion a filled slot never changes."""
    cfg = ModelConfig(L=2, D=256, Hq=4, Hkv=2, hd=64, E=8, k=2, F=128, V=512, act="f32", expert="f32")
    seed, B, P, N, S, n_canvases = 23, 2, 5, 16, 6, 2
    mask_id = cfg.V - 1 if sampler == "masked" else None
    pair = Pair(cfg, seed, scale_lm=12.0)
    prompt = synth.tokens(cfg.V, (B, P), seed, name="prompt")
    commits, touched, lens, ks, vs, kept, used = oracle_generate(
        pair.om, cfg, prompt.numpy(), n_canvases, N, S, tau, seed, sampler, mask_id, early_exit)
    cap = P + n_canvases * N
    kv = pair.gm.kv_cache(B, cap, device=DEV)
    ws = pair.gm.workspace(B * N, cap, device=DEV)
    res = driver.generate(pair.gm, kv, prompt.to(DEV), n_canvases, N, S, tau, seed, ws, sampler=sampler,
                          mask_id=mask_id, early_exit=early_exit)
    torch.cuda.synchronize()
    assert res.passes == used
    for c in range(n_canvases):
        np.testing.assert_array_equal(host(res.canvases[c]), commits[c], err_msg=f"canvas {c}")
    np.testing.assert_array_equal(host(res.touched), touched)
    assert res.lens == [int(x) for x in lens]
    if sampler == "masked":
        assert all((cm != mask_id).all() for cm in commits)   # the last pass fills every slot
    print(sampler, tau, early_exit, "passes", used, "kept", np.round(np.mean(kept), 3), flush=True)


@pytest.mark.parametrize("B,N", [(1, 256), (3, 37), (8, 256), (64, 5)])
def test_canvas_update_matches_oracle(B, N):
    """dg_canvas_update, both samplers, bit-exact with the oracle, with the
    per-request counts equal to brute-force counts."""
    from block_diffusion_lm_denoise_amd import dgpass
    V, tau, seed, mask_id = 1000, 0.4, 77, 999
    rng = np.random.default_rng(B * 1000 + N)
    canvas = rng.integers(0, V, (B, N)).astype(np.int32)
    canvas[rng.random((B, N)) < 0.5] = mask_id
    argmax = rng.integers(0, V, (B, N)).astype(np.int32)
    conf = rng.random((B, N)).astype(np.float32)
    conf[0, 0] = np.nan
    pos0 = rng.integers(0, 5000, B).astype(np.int32)
    ch = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    ml = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    dam = torch.from_numpy(argmax).to(DEV)
    dcf = torch.from_numpy(conf).to(DEV)
    # uniform
    g = torch.from_numpy(canvas).to(DEV)
    dgpass.canvas_update(g, dam, dcf, dict(tau=tau, seed=seed, pass_tag=3, pos0=pos0, changed=ch,
                                           masked_left=ml), V)
    o = oracle.renoise(canvas, argmax, conf, tau, seed, 3, pos0, V)
    np.testing.assert_array_equal(host(g), o)
    np.testing.assert_array_equal(host(ch), (o != canvas).sum(1))
    np.testing.assert_array_equal(host(ml), np.zeros(B, np.int32))
    # masked, a middle pass and the last pass
    for final in (False, True):
        g = torch.from_numpy(canvas).to(DEV)
        dgpass.canvas_update(g, dam, dcf, dict(sampler="masked", mask_id=mask_id, tau=tau,
                                               final_pass=final, changed=ch, masked_left=ml), V)
        o, och, oml = oracle.unmask(canvas, argmax, conf, tau, mask_id, final_pass=final)
        np.testing.assert_array_equal(host(g), o)
        np.testing.assert_array_equal(host(ch), och)
        np.testing.assert_array_equal(host(ml), oml)
    # initialisation: uniform noise (tag 0) or the mask token everywhere
    g = torch.zeros(B, N, dtype=torch.int32, device=DEV)
    dgpass.canvas_update(g, None, None, dict(tau=tau, seed=seed, pass_tag=0, pos0=pos0), V)
    np.testing.assert_array_equal(host(g), oracle.renoise(np.zeros((B, N), np.int32), None, None, tau, seed,
                                                          0, pos0, V))
    dgpass.canvas_update(g, None, None, dict(sampler="masked", mask_id=mask_id), V)
    assert (host(g) == mask_id).all()


def test_fused_masked_update_equals_separate_call():
    """The pass's last kernel doing the masked update (and its counts) gives
    the tokens and counts of the separate call after the pass."""
    from block_diffusion_lm_denoise_amd import dgpass
    cfg = ModelConfig(L=1, D=256, Hq=4, Hkv=2, hd=64, E=8, k=2, F=128, V=512, act="bf16", expert="bf16")
    pair = Pair(cfg, 24, scale_lm=12.0)
    B, N, P = 2, 40, 9
    oks, ovs, oln, kv = pair.caches(B, P + N, [P, 3], 24)
    rng = np.random.default_rng(24)
    canvas = rng.integers(0, cfg.V, (B, N)).astype(np.int32)
    canvas[rng.random((B, N)) < 0.6] = cfg.V - 1
    ws = pair.gm.workspace(B * N, P + N, device=DEV)
    outs = []
    for fused in (True, False):
        cv = torch.from_numpy(canvas).to(DEV)
        am = torch.empty(B, N, dtype=torch.int32, device=DEV)
        cf = torch.empty(B, N, dtype=torch.float32, device=DEV)
        ch = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        ml = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        args = dict(sampler="masked", mask_id=cfg.V - 1, tau=0.3, changed=ch, masked_left=ml)
        if fused:
            pair.gm.denoise_pass_next(kv, cv, am, cf, ws, renoise=args)
        else:
            pair.gm.denoise_pass(kv, cv, am, cf, ws)
            dgpass.canvas_update(cv, am, cf, args, cfg.V)
        torch.cuda.synchronize()
        outs.append((host(cv), host(am), host(cf), host(ch), host(ml)))
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    assert (outs[0][4] >= 0).all() and (outs[0][3] >= 0).all()


@pytest.mark.parametrize("sampler,tau", [("uniform", 0.5), ("masked", 0.0)])
def test_early_exit_stops_a_converged_canvas(sampler, tau):
    """Uniform noise: a model built to have a fixed point -- layers that
    barely move the residual (output projections scaled down) and a head tied
    to the embedding, so each slot predicts its own token with high
    confidence -- converges after the first pass (every slot kept, nothing
    changes).  Masked diffusion with tau 0 fills every slot at the first
    update (the planted head predicts tokens other than the mask).  The GPU
    stops after the same pass as the oracle loop."""
    cfg = ModelConfig(L=1, D=256, Hq=4, Hkv=2, hd=64, E=8, k=2, F=128, V=512, act="f32", expert="f32")
    seed, B, P, N, S, n_canvases = 25, 2, 5, 16, 6, 2
    if sampler == "uniform":
        w = synth.make_weights(cfg, seed, gain="ones")
        w["lm"] = (w["emb"] * 60.0).contiguous()
        for lw in w["layers"]:
            lw["wo"] = (lw["wo"] * 1e-3).contiguous()
            lw["wd"] = (lw["wd"] * 1e-3).contiguous()
        pair = Pair(cfg, seed, weights=w)
    else:
        pair = Pair(cfg, seed, scale_lm=12.0)
    mask_id = cfg.V - 1 if sampler == "masked" else None
    prompt = synth.tokens(cfg.V, (B, P), seed, name="prompt")
    commits, touched, lens, _, _, kept, used = oracle_generate(
        pair.om, cfg, prompt.numpy(), n_canvases, N, S, tau, seed, sampler, mask_id, True)
    kv = pair.gm.kv_cache(B, P + n_canvases * N, device=DEV)
    ws = pair.gm.workspace(B * N, P + n_canvases * N, device=DEV)
    res = driver.generate(pair.gm, kv, prompt.to(DEV), n_canvases, N, S, tau, seed, ws, sampler=sampler,
                          mask_id=mask_id, early_exit=True)
    torch.cuda.synchronize()
    assert res.passes == used and all(1 <= u < S for u in used), (res.passes, used)
    for c in range(n_canvases):
        np.testing.assert_array_equal(host(res.canvases[c]), commits[c])
    np.testing.assert_array_equal(host(res.touched), touched)
    print(sampler, "early exit after passes", used, flush=True)


@pytest.mark.parametrize("sampler,stop", [("uniform", (1, 2)), ("uniform", (0, 0)), ("masked", (1, 1))])
def test_stop_and_resume_reproduces_the_run(sampler, stop):
    """The state between two passes is (KV cache with its lengths, canvas,
    canvas and pass index, seed): a run stopped before pass p of canvas c
    and resumed from a copy of that state commits the same canvases, with
    the same coverage and the same cache, as the uninterrupted run
    (explainer "DiffusionGemma", "Long-form text: chaining canvases": the
    cache carries everything earlier canvases left)."""
    cfg = ModelConfig(L=2, D=256, Hq=4, Hkv=2, hd=64, E=8, k=2, F=128, V=512, act="bf16", expert="bf16")
    seed, tau, B, P, N, S, n_canvases = 31, 0.5, 2, 6, 16, 4, 3
    mask_id = cfg.V - 1 if sampler == "masked" else None
    pair = Pair(cfg, seed, scale_lm=12.0)
    prompt = synth.tokens(cfg.V, (B, P), seed, name="prompt").to(DEV)
    cap = P + n_canvases * N
    ws = pair.gm.workspace(B * N, cap, device=DEV)
    kw = dict(sampler=sampler, mask_id=mask_id)

    kv = pair.gm.kv_cache(B, cap, device=DEV)
    whole = driver.generate(pair.gm, kv, prompt, n_canvases, N, S, tau, seed, ws, **kw)

    kv1 = pair.gm.kv_cache(B, cap, device=DEV)
    first = driver.generate(pair.gm, kv1, prompt, n_canvases, N, S, tau, seed, ws, stop=stop, **kw)
    assert first.state is not None and len(first.canvases) == stop[0]
    # the saved state: a copy of the cache and its lengths, the canvas, (c, p)
    kv2 = pair.gm.kv_cache(B, cap, device=DEV)
    for l in range(cfg.L):
        kv2.k[l].copy_(kv1.k[l])
        kv2.v[l].copy_(kv1.v[l])
    kv2.lens[:] = kv1.lens
    del kv1
    rest = driver.generate(pair.gm, kv2, None, n_canvases, N, S, tau, seed, ws, prefill_prompt=False,
                           start=first.state, **kw)
    torch.cuda.synchronize()

    commits = first.canvases + rest.canvases
    assert len(commits) == n_canvases
    for c in range(n_canvases):
        np.testing.assert_array_equal(host(commits[c]), host(whole.canvases[c]), err_msg=f"canvas {c}")
    c0, p0 = stop
    wt, ft, rt = host(whole.touched), host(first.touched), host(rest.touched)
    np.testing.assert_array_equal(ft[:c0], wt[:c0])
    np.testing.assert_array_equal(ft[c0, :p0], wt[c0, :p0])
    np.testing.assert_array_equal(rt[c0, p0:], wt[c0, p0:])
    np.testing.assert_array_equal(rt[c0 + 1:], wt[c0 + 1:])
    assert rest.lens == whole.lens
    for l in range(cfg.L):
        n = max(whole.lens)
        assert torch.equal(kv2.k[l][:, :, :n], kv.k[l][:, :, :n])
        assert torch.equal(kv2.v[l][:, :, :n], kv.v[l][:, :, :n])
