"""Oracle layer pieces pinned to library routines (torch CPU float64) and
special cases: RMSNorm, projections, router, top-k, permutation, experts,
combine, LM head, argmax and confidence.

Pages: newsletter comment under "A Visual Guide to DiffusionGemma" (all
canvas tokens go through the router; a pass reads the union of the selected
experts), course page "Module 12. Diffusion Language Models", dense-8B
exercise (different positions select different experts), explainer
"DiffusionGemma", "Uniform State Diffusion" (confidence decides re-noise).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from block_diffusion_lm_denoise_amd import synth
from helpers import act_to_f64, max_rel, oracle_model, prefilled, rnd, t64, tiny_cfg

TAPS = ("qkv", "attn", "x1", "u2", "router", "ids", "gates", "counts", "offsets", "perm", "hmid",
        "yexp", "xout", "uf", "logits")


def _run(cfg, seed=0, P=7, N=10, B=1, scale_lm=1.0, inject=None):
    model, w = oracle_model(cfg, seed=seed, scale_lm=scale_lm)
    ks, vs, ln = prefilled(model, cfg, B, P, cap=P + 4, seed=seed)
    canvas = synth.tokens(cfg.V, (B, N), seed, "canvas").numpy()
    am, cf, t = model.denoise_pass(ks, vs, ln, canvas, taps=TAPS, inject_router=inject)
    return model, w, canvas, am, cf, t


def _f(t, name, act):
    return torch.tensor(act_to_f64(t[name], act))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_norms_projections_residual_match_torch(act):
    cfg = tiny_cfg(L=1, act=act, expert=act)
    _, w, canvas, _, _, t = _run(cfg, seed=1)
    lw = w["layers"][0]
    x = t64(w["emb"])[torch.tensor(canvas.ravel(), dtype=torch.long)]
    u = rnd(Fn.rms_norm(x, (cfg.D,), weight=t64(lw["g1"]), eps=cfg.eps), act)
    wqkv = torch.cat([t64(lw["wq"]), t64(lw["wk"]), t64(lw["wv"])])
    qkv = rnd(Fn.linear(u, wqkv), act)
    tol = 1e-6 if act == "f32" else 1e-2
    assert max_rel(_f(t, "qkv", act)[0], qkv) < tol
    # residual after attention, from the oracle's own attention output
    x1 = rnd(x + Fn.linear(_f(t, "attn", act)[0], t64(lw["wo"])), act)
    assert max_rel(_f(t, "x1", act)[0], x1) < tol
    u2 = rnd(Fn.rms_norm(_f(t, "x1", act)[0], (cfg.D,), weight=t64(lw["g2"]), eps=cfg.eps), act)
    assert max_rel(_f(t, "u2", act)[0], u2) < tol
    r = Fn.linear(_f(t, "u2", act)[0], t64(lw["wr"])).to(torch.float32)
    np.testing.assert_allclose(t["router"][0], r.numpy(), rtol=1e-6, atol=1e-7)


def test_topk_gates_permutation_match_sorts():
    cfg = tiny_cfg(L=2, E=16, k=4)
    _, _, _, _, _, t = _run(cfg, seed=2, N=25)
    for l in range(cfg.L):
        r = t["router"][l]
        # top-k = the first k of a stable descending sort (lower index wins ties)
        order = np.argsort(-r, axis=1, kind="stable")[:, :cfg.k]
        np.testing.assert_array_equal(t["ids"][l], order)
        sel = torch.tensor(np.take_along_axis(r, order, 1), dtype=torch.float64)
        np.testing.assert_allclose(t["gates"][l], torch.softmax(sel, 1).numpy(), rtol=1e-6)
        flat = t["ids"][l].ravel()
        np.testing.assert_array_equal(t["perm"][l], np.argsort(flat, kind="stable"))
        np.testing.assert_array_equal(t["counts"][l], np.bincount(flat, minlength=cfg.E))
        np.testing.assert_array_equal(t["offsets"][l], np.concatenate([[0], np.cumsum(t["counts"][l])]))
        assert t["offsets"][l][-1] == 25 * cfg.k


def test_topk_ties_go_to_lower_expert_index():
    cfg = tiny_cfg(E=8, k=3)
    N = 4
    inj = np.zeros((1, N, 8), np.float32)
    inj[0, 0] = [1, 2, 2, 0, 2, -1, 5, 0]      # tie at 2 among 1, 2, 4 -> 6, 1, 2
    inj[0, 1] = [0, 0, 0, 0, 0, 0, 0, 0]        # all equal -> 0, 1, 2
    inj[0, 2] = [3, 1, 3, 1, 3, 9, 3, 1]        # 5, then ties at 3 -> 0, 2
    inj[0, 3] = [-1, -1, -2, -1, 7, -1, 7, 7]   # 4, 6, 7
    _, _, _, _, _, t = _run(cfg, seed=3, N=N, inject=inj)
    np.testing.assert_array_equal(t["ids"][0], [[6, 1, 2], [0, 1, 2], [5, 0, 2], [4, 6, 7]])
    np.testing.assert_array_equal(t["router"][0], inj[0])


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_experts_per_slot_match_torch(act):
    cfg = tiny_cfg(L=1, act=act, expert=act, E=6, k=2)
    _, w, _, _, _, t = _run(cfg, seed=4, N=12)
    lw = w["layers"][0]
    u2 = _f(t, "u2", act)[0]
    h_all = _f(t, "hmid", act)[0]
    y_all = _f(t, "yexp", act)[0]
    tol = 1e-6 if act == "f32" else 1e-2
    for tk in range(12):
        for j in range(cfg.k):
            e = int(t["ids"][0, tk, j])
            a = Fn.linear(u2[tk], t64(lw["wg"][e]))
            c = Fn.linear(u2[tk], t64(lw["wu"][e]))
            h = rnd(Fn.silu(a) * c, act)
            assert max_rel(h_all[tk, j], h) < tol
            y = rnd(Fn.linear(h_all[tk, j], t64(lw["wd"][e])), act)
            assert max_rel(y_all[tk, j], y) < tol


def test_single_expert_is_a_dense_swiglu_ffn():
    """E = k = 1: the gate is exactly 1 and the MoE is one SwiGLU FFN."""
    cfg = tiny_cfg(L=1, E=1, k=1)
    _, w, _, _, _, t = _run(cfg, seed=5)
    lw = w["layers"][0]
    np.testing.assert_array_equal(t["gates"][0], np.ones_like(t["gates"][0]))
    x1, u2 = _f(t, "x1", "f32")[0], _f(t, "u2", "f32")[0]
    h = rnd(Fn.silu(Fn.linear(u2, t64(lw["wg"][0]))) * Fn.linear(u2, t64(lw["wu"][0])), "f32")
    y = rnd(Fn.linear(h, t64(lw["wd"][0])), "f32")
    assert max_rel(_f(t, "xout", "f32")[0], rnd(x1 + y, "f32")) < 1e-6


def test_all_experts_selected_is_a_dense_softmax_mixture():
    """k = E: a dense gating matrix softmax(r) over every expert."""
    cfg = tiny_cfg(L=1, E=4, k=4)
    _, w, _, _, _, t = _run(cfg, seed=6)
    lw = w["layers"][0]
    x1, u2 = _f(t, "x1", "f32")[0], _f(t, "u2", "f32")[0]
    G = torch.softmax(torch.tensor(t["router"][0], dtype=torch.float64), dim=1)   # [N, E]
    ys = []
    for e in range(cfg.E):
        h = rnd(Fn.silu(Fn.linear(u2, t64(lw["wg"][e]))) * Fn.linear(u2, t64(lw["wu"][e])), "f32")
        ys.append(rnd(Fn.linear(h, t64(lw["wd"][e])), "f32"))
    Y = torch.stack(ys, 1)                                                       # [N, E, D]
    ref = rnd(x1 + torch.einsum("ne,ned->nd", G, Y), "f32")
    assert max_rel(_f(t, "xout", "f32")[0], ref) < 1e-6


def test_fp8_scale_applies_after_accumulation():
    """fp8 codes with per-expert scales equal the dequantised fp32 weights."""
    cfg8 = tiny_cfg(L=1, act="f32", expert="fp8", E=4, k=2)
    model8, w8 = oracle_model(cfg8, seed=7)
    w32 = dict(w8)
    lw = dict(w8["layers"][0])
    for i, n in enumerate(("wg", "wu", "wd")):
        lw[n] = lw[n].to(torch.float32) * lw["escale"][:, i][:, None, None]
    lw["escale"] = None
    w32["layers"] = [lw]
    cfg32 = tiny_cfg(L=1, act="f32", expert="f32", E=4, k=2)
    model32, _ = oracle_model(cfg32, weights=w32)
    canvas = synth.tokens(cfg8.V, (1, 9), 7, "canvas").numpy()
    ln = np.zeros(1, np.int32)
    a8, c8, t8 = model8.denoise_pass([], [], ln, canvas, taps=("xout", "hmid", "logits"))
    a32, c32, t32 = model32.denoise_pass([], [], ln, canvas, taps=("xout", "hmid", "logits"))
    assert max_rel(t8["hmid"], t32["hmid"]) < 1e-5
    assert max_rel(t8["xout"], t32["xout"]) < 1e-5
    assert max_rel(t8["logits"], t32["logits"]) < 1e-5


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_head_argmax_confidence_match_library(act):
    cfg = tiny_cfg(L=2, act=act, expert=act, V=300)
    _, w, _, am, cf, t = _run(cfg, seed=8, scale_lm=25.0)
    uf = rnd(Fn.rms_norm(_f(t, "xout", act)[1], (cfg.D,), weight=t64(w["gf"]), eps=cfg.eps), act)
    tol = 1e-6 if act == "f32" else 1e-2
    assert max_rel(_f(t, "uf", act), uf) < tol
    lg = Fn.linear(_f(t, "uf", act), t64(w["lm"]))
    np.testing.assert_allclose(t["logits"], lg.to(torch.float32).numpy(), rtol=1e-6, atol=1e-6)
    # argmax: first maximum of the fp32 logits
    np.testing.assert_array_equal(am.ravel(), np.argmax(t["logits"], axis=1))
    # confidence: softmax probability of the maximum
    ref = torch.exp(lg.max(1).values - torch.logsumexp(lg, 1)).numpy()
    np.testing.assert_allclose(cf.ravel(), ref, rtol=1e-6)
    # the planted head spreads confidence across the re-noise threshold
    assert cf.min() < 0.5 < cf.max()


def test_argmax_ties_pick_lowest_index():
    """Two identical head rows tie exactly; the lower vocabulary index wins."""
    cfg = tiny_cfg(L=1, V=64)
    model, w = oracle_model(cfg, seed=9, scale_lm=30.0)
    ln = np.zeros(1, np.int32)
    canvas = synth.tokens(cfg.V, (1, 6), 9, "canvas").numpy()
    am, _, t = model.denoise_pass([], [], ln, canvas, taps=("logits",))
    w2 = dict(w)
    lm = w["lm"].clone()
    lo = np.minimum(am.ravel(), 5)
    for tk in range(6):
        # copy the winning row to a lower index; the tie must resolve downwards
        lm[int(lo[tk])] = lm[int(am.ravel()[tk])]
    w2["lm"] = lm
    m2, _ = oracle_model(cfg, weights=w2)
    am2, _, t2 = m2.denoise_pass([], [], ln, canvas, taps=("logits",))
    np.testing.assert_array_equal(am2.ravel(), np.argmax(t2["logits"], axis=1))


def test_expert_coverage_follows_closed_form_under_random_routing():
    """With i.i.d. router logits each token's top-k is a uniform k-subset, so the
    expected number of experts touched is E (1 - (1 - k/E)^BN)
    (newsletter comment: a 256-token canvas lights up most experts)."""
    cfg = tiny_cfg(L=1, E=8, k=2, D=32, F=8, V=64)
    model, _ = oracle_model(cfg, seed=10)
    rng = np.random.default_rng(10)
    ln = np.zeros(1, np.int32)
    canvas = synth.tokens(cfg.V, (1, 16), 10, "canvas").numpy()
    touched = []
    for _ in range(600):
        inj = rng.standard_normal((1, 16, 8)).astype(np.float32)
        _, _, t = model.denoise_pass([], [], ln, canvas, taps=("counts",), inject_router=inj)
        touched.append(int((t["counts"][0] > 0).sum()))
    expect = 8 * (1 - (1 - 2 / 8) ** 16)
    sd = np.std(touched) / np.sqrt(len(touched))
    assert abs(np.mean(touched) - expect) < 5 * max(sd, 0.005), (np.mean(touched), expect)
    # 128 experts, top-8, 256 tokens: an expert stays untouched with prob 6.7e-8
    cfg2 = tiny_cfg(L=1, E=128, k=8, D=32, F=8, V=64)
    m2, _ = oracle_model(cfg2, seed=11)
    cv = synth.tokens(cfg2.V, (1, 256), 11, "canvas").numpy()
    inj = rng.standard_normal((1, 256, 128)).astype(np.float32)
    _, _, t = m2.denoise_pass([], [], ln, cv, taps=("counts",), inject_router=inj)
    assert (t["counts"][0] > 0).sum() == 128
