"""Autoregressive decoding step (dg_decode_step) on the GPU against the oracle.

Course page "Module 12. Diffusion Language Models", break-even solution:
autoregressive decoding emits one token per pass over the weights; the
canvas pass is weighed against that step.  The oracle computes a step as what
it is by definition: the new token's K/V appended to the cache (a causal
prefill of one token) and the head over that token's final state, which is a
denoising pass over a one-slot canvas (its one query sees the prefix and
itself: causal for the last position).
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_denoise_amd import synth
from block_diffusion_lm_denoise_amd.configs import WORKLOADS, ModelConfig
from gpu_helpers import DEV, TOL, Pair, argmax_report, f64, host, max_rel, to_torch_act

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    base = dict(L=2, D=256, Hq=4, Hkv=2, hd=64, E=8, k=2, F=128, V=512, act="bf16", expert="bf16")
    base.update(kw)
    return ModelConfig(**base)


def _step_and_compare(pair, kv, oks, ovs, oln, tokens, label):
    """One step on both sides from identical caches; the GPU's head also runs
    on the oracle's final-norm rows for the argmax bar."""
    cfg = pair.cfg
    B = len(tokens)
    o = pair.om.denoise_pass(oks, ovs, oln, np.asarray(tokens, np.int32).reshape(B, 1),
                             taps=("uf", "logits"))
    pair.om.kv_prefill(oks, ovs, oln, np.asarray(tokens, np.int32).reshape(B, 1))
    ws = pair.gm.workspace(B, int(kv.lens.max()) + 1, device=DEV)
    res = {}
    for inject in (True, False):
        if inject:   # the cache update is checked on the free step below
            kv2 = pair.gm.kv_cache(B, kv.cap, device=DEV)
            for l in range(cfg.L):
                kv2.k[l].copy_(kv.k[l])
                kv2.v[l].copy_(kv.v[l])
            kv2.lens[:] = kv.lens
            run_kv = kv2
        else:
            run_kv = kv
        am = torch.empty(B, dtype=torch.int32, device=DEV)
        cf = torch.empty(B, dtype=torch.float32, device=DEV)
        from block_diffusion_lm_denoise_amd import dgpass
        tp = dgpass.make_taps(cfg, B, ("uf", "logits"), device=DEV)
        pair.gm.decode_step(run_kv, torch.tensor(tokens, dtype=torch.int32, device=DEV), am, cf, ws,
                            taps=tp, inject_uf=to_torch_act(o[2]["uf"], cfg.act).to(DEV) if inject else None)
        torch.cuda.synchronize()
        rep, fails = {}, []
        gt = {n: host(t) for n, t in tp.items()}
        argmax_report(rep, fails, o[0], o[1], host(am), host(cf), o[2], gt, np.ones(B, bool),
                      assert_argmax=inject or cfg.act == "f32")
        rep["uf"] = max_rel(f64(gt["uf"], cfg.act), f64(o[2]["uf"], cfg.act))
        for n in ("uf", "logits", "conf"):
            if rep.get(n, 0.0) >= TOL[cfg.act]:
                fails.append(f"{n} max-rel {rep[n]:.3e}")
        assert not fails, (label, inject, fails, rep)
        res["inject" if inject else "free"] = rep
    np.testing.assert_array_equal(kv.lens, oln)
    for l in range(cfg.L):
        for b in range(B):
            n = int(oln[b])
            for g_, o_ in ((kv.k[l], oks[l]), (kv.v[l], ovs[l])):
                r = max_rel(f64(host(g_[b, :, :n]), cfg.act), f64(o_[b, :, :n], cfg.act))
                assert r < TOL[cfg.act], (label, l, b, r)
    print(label, res, flush=True)
    return res


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_decode_steps_ragged_batch(act):
    cfg = _cfg(act=act, expert=act)
    pair = Pair(cfg, 51, scale_lm=10.0)
    lens = [20, 0, 7]
    oks, ovs, oln, kv = pair.caches(3, 40, lens, 51)
    # three steps, teacher-forced on the oracle's tokens
    toks = synth.tokens(cfg.V, (3,), 51, "first").numpy().tolist()
    for step in range(3):
        o = pair.om.denoise_pass(oks, ovs, oln, np.asarray(toks, np.int32).reshape(3, 1))
        _step_and_compare(pair, kv, oks, ovs, oln, toks, f"{act} step {step}")
        toks = o[0].ravel().tolist()


def test_decode_step_full_width_prefix1024():
    """One step of one request at the 1024-prefix layer's full size."""
    wl = WORKLOADS["layer_p1024"]
    pair = Pair(wl.model, wl.seed, gain="ones")
    oks, ovs, oln, kv = pair.caches(1, wl.P + 4, [wl.P], wl.seed, synthetic=True)
    tok = synth.tokens(wl.model.V, (1,), wl.seed, "step").numpy().tolist()
    _step_and_compare(pair, kv, oks, ovs, oln, tok, "layer_p1024 step")


def test_decode_chain_fp32_equals_oracle_chain():
    """Greedy autoregressive generation of six tokens, each step fed its own
    previous output: fp32 tokens equal the oracle's chain exactly."""
    wl = WORKLOADS["tiny_fp32"]
    pair = Pair(wl.model, wl.seed, gain="ones", scale_lm=10.0)
    cap = wl.P + 8
    oks, ovs, oln, kv = pair.caches(1, cap, [wl.P], wl.seed)
    ws = pair.gm.workspace(1, cap, device=DEV)
    tok_o = tok_g = [int(synth.tokens(wl.model.V, (1,), 3, "start")[0])]
    out_o, out_g = [], []
    am = torch.empty(1, dtype=torch.int32, device=DEV)
    cf = torch.empty(1, dtype=torch.float32, device=DEV)
    for _ in range(6):
        o = pair.om.denoise_pass(oks, ovs, oln, np.asarray(tok_o, np.int32).reshape(1, 1))
        pair.om.kv_prefill(oks, ovs, oln, np.asarray(tok_o, np.int32).reshape(1, 1))
        tok_o = [int(o[0][0, 0])]
        out_o.append(tok_o[0])
        pair.gm.decode_step(kv, torch.tensor(tok_g, dtype=torch.int32, device=DEV), am, cf, ws)
        torch.cuda.synchronize()
        tok_g = [int(am[0])]
        out_g.append(tok_g[0])
    assert out_g == out_o
    np.testing.assert_array_equal(kv.lens, oln)
